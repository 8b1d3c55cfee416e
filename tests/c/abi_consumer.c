/*
 * A plain C11 caller of the library's C ABI (include/fa.h): it compiles
 * against the header as C, links against libfa.so, and exercises the entry
 * points whose outcome is decided on the host before any launch (status
 * strings, the version, workspace sizing, and argument validation), so it
 * runs without a GPU. Prints "abi consumer ok" and exits 0 on success.
 */
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int failures = 0;

static void expect(int cond, const char* what) {
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

int main(void) {
    static _Alignas(256) unsigned char buf[4096];
    void* p = buf;
    float* f = (float*)(void*)buf;
    fa_fwd_options opt;
    size_t ws;

    expect(fa_version() != NULL && strlen(fa_version()) > 0, "fa_version");
    expect(strlen(fa_status_string(FA_OK)) > 0, "status string of FA_OK");
    expect(strlen(fa_status_string(FA_ERR_UNSUPPORTED)) > 0, "status string of FA_ERR_UNSUPPORTED");

    /* empty problems are valid and enqueue nothing, pointers or not */
    expect(fa_fwd(NULL, NULL, NULL, NULL, NULL, 0, 2, 2, 128, 128, 1, 0.1f, NULL, NULL) == FA_OK, "empty forward");
    expect(fa_bwd_workspace_size(0, 2, 2, 128, 128, 1, 0) == 0, "empty workspace size");

    /* validation on the host: nothing is launched for these */
    expect(fa_fwd(NULL, p, p, p, f, 1, 2, 2, 64, 128, 0, 0.1f, NULL, NULL) == FA_ERR_INVALID_ARGUMENT, "null q");
    expect(fa_fwd(p, p, p, p, f, 1, 3, 2, 64, 128, 0, 0.1f, NULL, NULL) == FA_ERR_INVALID_ARGUMENT, "Hq % Hkv");
    expect(fa_fwd(p, p, p, p, f, 1, 2, 2, 64, 96, 0, 0.1f, NULL, NULL) == FA_ERR_UNSUPPORTED, "d = 96");
    expect(fa_fwd(p, p, p, p, f, 1, 2, 2, 64, 128, 0, -1.0f, NULL, NULL) == FA_ERR_INVALID_ARGUMENT, "scale < 0");
    opt.exp_mode = 7;
    opt.rescale_tau = 32.0f;
    opt.lpt_order = 1;
    expect(fa_fwd_ex(p, p, p, p, f, 1, 2, 2, 64, 128, 0, 0.1f, NULL, &opt, NULL) == FA_ERR_INVALID_ARGUMENT,
           "bad exp mode");

    /* the backward's workspace grows with the problem and the call checks it */
    ws = fa_bwd_workspace_size(2, 16, 16, 8192, 128, 1, 0);
    expect(ws > 0 && ws >= fa_bwd_workspace_size(1, 16, 16, 8192, 128, 1, 0), "workspace size grows with B");
    expect(fa_bwd(p, p, p, p, f, p, p, p, p, 2, 16, 16, 8192, 128, 1, 0.1f, NULL, NULL, 0, NULL) == FA_ERR_WORKSPACE,
           "missing workspace");
    expect(fa_bwd_noalloc_max_workspace() > 0, "no-alloc workspace limit");

    if (failures) return 1;
    printf("abi consumer ok\n");
    return 0;
}
