/* A plain C99 consumer of include/vpa.h: it links against libvpa and makes
 * calls that the library answers on the host (slot counts, workspace sizes,
 * rejected arguments, empty batches), so it runs without a GPU.  It prints
 * one line per check and exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "vpa.h"

static int check(int ok, const char* what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    return ok ? 0 : 1;
}

int main(void) {
    vpa_vocab v = {200064, 25008, 8};
    vpa_vocab bad = {0, 1, 1};
    int32_t dummy_ids[4];
    vpa_stat* no_stats = NULL;
    if (check(vpa_stats_slots(25008, 8, 8192) == 4, "slots at 8192-blocks"))
        return 1;
    if (check(vpa_stats_slots(25008, 8, 1024) == 26, "slots at 1024-blocks"))
        return 1;
    if (check(vpa_top_tokens_workspace(v, 4096, 8192) > 0, "workspace size"))
        return 1;
    if (check(vpa_block_stats((const void*)16, VPA_BF16, 200064, bad, 0, 1, NULL, 4, 4, 8192,
                              no_stats, NULL) == VPA_ERR_INVALID,
              "invalid vocabulary rejected"))
        return 1;
    if (check(strlen(vpa_last_error()) > 0, "error message set"))
        return 1;
    if (check(vpa_block_stats((const void*)16, (vpa_dtype)9, 200064, v, 0, 8, NULL, 4, 4, 8192,
                              no_stats, NULL) == VPA_ERR_UNSUPPORTED,
              "unknown dtype rejected"))
        return 1;
    if (check(vpa_combine_stats(NULL, 8, 0, 4, NULL, dummy_ids, NULL, NULL, NULL) == VPA_OK,
              "empty batch is a no-op"))
        return 1;
    return 0;
}
