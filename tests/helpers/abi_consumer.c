/* A plain C11 caller of the library: it includes include/tk.h, links
 * libtk.so and exercises what a C program sees without a GPU -- the error
 * codes and per-thread message of the host-side argument checks, the T == 0
 * no-op, the workspace size queries and the layout of tk_route_opts.  Every
 * failing call below is rejected before anything is launched, so no pointer
 * passed here is dereferenced.  Prints one "name value" line per check for
 * the test that builds and runs it. */
#include "tk.h"

#include <stddef.h>
#include <stdio.h>
#include <string.h>

static void report(const char* name, tk_status st)
{
    const char* msg = tk_last_error();
    printf("%s %d %d\n", name, (int)st, msg != NULL && msg[0] != '\0');
}

int main(void)
{
    void* fake = (void*)(uintptr_t)0x10000;   /* aligned, never dereferenced */
    int32_t* ifake = (int32_t*)fake;
    float* ffake = (float*)fake;

    printf("initial_error_empty %d\n", tk_last_error()[0] == '\0');
    printf("opts_size %zu\n", sizeof(tk_route_opts));
    printf("opts_scale_offset %zu\n", offsetof(tk_route_opts, route_scale));

    tk_route_opts opts = {TK_SCORE_SIGMOID, 8, 4, 2, 1, 2.5f};
    report("route_null_opts", tk_route(ffake, NULL, 8192, 256, 8, NULL, ifake, ffake, NULL));
    report("route_too_many_experts",
           tk_route(ffake, NULL, 64, TK_MAX_EXPERTS + 1, 8, &opts, ifake, ffake, NULL));
    report("reduce_bad_h", tk_reduce(fake, 16, ifake, ffake, 2, 8, 7, fake, NULL));
    report("reduce_no_tokens", tk_reduce(NULL, 0, NULL, NULL, 0, 8, 7168, NULL, NULL));
    report("expand_bad_mode", tk_expand_quant(fake, 2, 256, 8, ifake, 7, fake, ffake, 16, NULL));

    printf("map_ws %zu\n", tk_map_workspace_bytes(8192, 8, 256));
    printf("balance_ws %zu\n", tk_balance_workspace_bytes(8192, 256));
    printf("quant_pc_ws %zu\n", tk_quant_workspace_bytes(8192, 7168, TK_QUANT_FP8_PER_CHANNEL));
    return 0;
}
