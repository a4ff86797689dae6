/* Plain C99 client of include/attn.h: compiles the header as C, links
 * libattn.so and makes only calls that are rejected (or are no-ops) before
 * any HIP call, so it runs without a GPU. Prints one line per check and
 * exits non-zero on the first unexpected status. */
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int expect(const char* what, attn_status got, attn_status want) {
    printf("%s: %s\n", what, attn_status_string(got));
    if (got != want) {
        printf("expected %s\n", attn_status_string(want));
        return 1;
    }
    return 0;
}

int main(void) {
    void* fake = (void*)(size_t)0x10000; /* aligned, never dereferenced */
    attn_varlen_dims vd = {2, 100, 60, 16, 8, 128};
    attn_varlen_dims empty = {0, 0, 0, 16, 8, 128};
    attn_varlen_dims bad_d = {2, 100, 60, 16, 8, 96};
    attn_paged_dims pd = {4, 16, 8, 128, 32, 64, 1000, 1024};
    attn_rope_tables short_tab = {(const float*)fake, (const float*)fake, 10};
    int fails = 0;
    fails += expect("fwd null dims", attn_fwd(NULL, fake, fake, fake, fake, 0.1f, fake, fake, NULL),
                    ATTN_ERR_INVALID_ARG);
    fails += expect("fwd head_dim 96", attn_fwd(&bad_d, fake, fake, fake, fake, 0.1f, fake, fake, NULL),
                    ATTN_ERR_UNSUPPORTED);
    fails += expect("fwd empty batch", attn_fwd(&empty, fake, fake, fake, fake, 0.1f, fake, fake, NULL),
                    ATTN_OK);
    fails += expect("bwd workspace 0",
                    attn_bwd(&vd, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, 0.1f,
                             fake, 0, NULL),
                    ATTN_ERR_WORKSPACE);
    fails += expect("bwd workspace size > 0", attn_bwd_workspace_bytes(&vd) > 0 ? ATTN_OK
                                                                          : ATTN_ERR_WORKSPACE,
                    ATTN_OK);
    fails += expect("decode block size 32",
                    attn_decode_paged(&pd, fake, fake, fake, fake, fake, fake, 0.1f, fake, 1 << 20,
                                      NULL),
                    ATTN_ERR_UNSUPPORTED);
    fails += expect("rope tables too short",
                    attn_rope(&vd, fake, fake, fake, NULL, 0, &short_tab, 0, NULL),
                    ATTN_ERR_INVALID_ARG);
    fails += expect("unknown status", strcmp(attn_status_string((attn_status)99),
                                             "ATTN_UNKNOWN_STATUS") == 0 ? ATTN_OK
                                                                          : ATTN_ERR_INVALID_ARG,
                    ATTN_OK);
    return fails ? 1 : 0;
}
