/* The library's host code (argument checks, workspace layouts, status strings) built with
 * AddressSanitizer and UndefinedBehaviorSanitizer, from the units compiled for the host
 * only (no device code, so nothing can be launched).  Every call below is refused or is
 * a pure host function: fake, never-dereferenced device addresses; problems that are
 * invalid, unsupported, misaligned, aliased or short of workspace; the workspace sizes of
 * every entry point over a grid of shapes, compared with their own layouts.  Exit status
 * 0 on success, 1 when a call returns something other than what is expected. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssd.h"

static int fails = 0;
#define EXPECT(cond)                                            \
    do {                                                        \
        if (!(cond)) {                                          \
            printf("line %d: expected %s\n", __LINE__, #cond); \
            ++fails;                                            \
        }                                                       \
    } while (0)

static ssd_problem prob(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q, int dtype,
                        int flags) {
    ssd_problem p;
    memset(&p, 0, sizeof(p));
    p.batch = b; p.seqlen = T; p.nheads = H; p.headdim = P; p.dstate = N; p.ngroups = G; p.chunk = Q;
    p.dtype = dtype; p.flags = flags;
    return p;
}

#define FAKE(k) ((void*)((uintptr_t)1 << 40 | (uintptr_t)(k) << 32))

int main(void) {
    const int64_t Ps[] = {16, 32, 64, 128}, Ns[] = {16, 32, 64, 128, 256}, Qs[] = {64, 128, 256};
    for (int dt = 0; dt < 2; ++dt)
        for (int ip = 0; ip < 4; ++ip)
            for (int in = 0; in < 5; ++in)
                for (int iq = 0; iq < 3; ++iq)
                    for (int diag = 0; diag < 2; ++diag)
                        for (int fl = 0; fl < 3; ++fl) {
                            const int flags = fl == 0 ? 0 : (fl == 1 ? SSD_SCHEDULE_SPLIT : SSD_SCHEDULE_FUSED);
                            ssd_problem p = prob(3, 1000 + 7 * ip, 8, Ps[ip], Ns[in], 2, Qs[iq], dt, flags);
                            ssd_workspace_layout L;
                            const int st = ssd_get_workspace_layout(&p, diag, &L);
                            EXPECT(st == SSD_OK);
                            EXPECT(ssd_workspace_bytes(&p, diag) == L.total_bytes);
                            EXPECT(L.total_bytes >= L.carry_off + L.carry_bytes);
                            (void)ssd_varlen_workspace_bytes(&p);
                            (void)ssd_bwd_workspace_bytes(&p);
                            (void)ssd_diag_bwd_workspace_bytes(&p);
                        }
    /* refused before any HIP call */
    ssd_problem p = prob(2, 300, 4, 64, 128, 2, 128, SSD_BF16, 0);
    const size_t wsb = ssd_workspace_bytes(&p, 0);
    EXPECT(ssd_scan_fwd(&p, NULL, FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, FAKE(6), wsb, NULL) ==
           SSD_ERR_NULL);
    EXPECT(ssd_scan_fwd(&p, FAKE(7), FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, FAKE(6), 16, NULL) ==
           SSD_ERR_WORKSPACE);
    EXPECT(ssd_scan_fwd(&p, (char*)FAKE(7) + 8, FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, FAKE(6),
                        wsb, NULL) == SSD_ERR_ALIGN);
    EXPECT(ssd_scan_fwd(&p, FAKE(7), FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(7), NULL, FAKE(6), wsb, NULL) ==
           SSD_ERR_ALIAS);
    EXPECT(ssd_scan_fwd_noalloc(&p, NULL, FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, NULL) ==
           SSD_ERR_NULL);
    ssd_problem big = prob(8, 4096, 80, 64, 128, 1, 256, SSD_BF16, SSD_SCHEDULE_SPLIT);
    EXPECT(ssd_scan_fwd_noalloc(&big, FAKE(7), FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, NULL) ==
           SSD_ERR_WORKSPACE);
    ssd_problem odd = prob(2, 300, 6, 64, 128, 4, 128, SSD_BF16, 0);
    EXPECT(ssd_workspace_bytes(&odd, 0) == 0);
    ssd_problem p48 = prob(2, 300, 4, 48, 128, 2, 128, SSD_BF16, 0);
    EXPECT(ssd_scan_fwd(&p48, FAKE(7), FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, FAKE(6), wsb,
                        NULL) == SSD_ERR_UNSUPPORTED);
    ssd_problem q = prob(2, 1, 4, 64, 128, 2, 64, SSD_BF16, 0);
    EXPECT(ssd_step(&q, FAKE(7), FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL) == SSD_ERR_NULL);
    EXPECT(ssd_scan_bwd(&p, NULL, FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, FAKE(8), FAKE(9),
                        FAKE(10), FAKE(11), FAKE(12), NULL, NULL, FAKE(6), 1 << 30, NULL) == SSD_ERR_NULL);
    EXPECT(ssd_scan_fwd_varlen(&p, NULL, FAKE(7), FAKE(1), FAKE(2), FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, FAKE(6),
                               1 << 30, NULL) == SSD_ERR_NULL);
    EXPECT(ssd_scan_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == SSD_ERR_NULL);
    for (int s = -1; s < 10; ++s) EXPECT(ssd_status_string(s) != NULL && strlen(ssd_status_string(s)) > 0);
    EXPECT(ssd_version() == SSD_VERSION);
    printf(fails ? "FAILED (%d)\n" : "OK\n", fails);
    return fails ? 1 : 0;
}
