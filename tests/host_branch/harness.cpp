// Test driver for the decode host branch on the CPU (no GPU, no HIP): runs host_pool_run, the
// product's host-side expert compute, on one layer step read from a file and writes the partial
// sums it produced. Built by the CPU tests with g++, plain and under the thread, address and
// undefined-behaviour sanitizers.
//
// Input (little-endian): int64 header[9] = T, k, H, I, wdtype, n_experts, E_bank, expert_bytes,
// reps; int32 host_ids[n_experts] (bank index of each host-list expert); int32 rewritten[T*k]
// (a slot >= 0, or -(1 + host-list index)); x [T*H] (f32 for wdtype 0, else bf16 bits);
// bank [E_bank * expert_bytes]. Output: float y[T*H*k].
// The job runs `reps` times on one worker pool (jobs arrive back to back, as in decode); every
// run must give bit-identical sums (exit 3 otherwise) and leave the GPU-side pairs' entries
// untouched (exit 4 otherwise).
#include "host_experts.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

static bool read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
    if (argc != 4) {
        std::fprintf(stderr, "usage: %s in.bin out.bin threads\n", argv[0]);
        return 2;
    }
    FILE* f = std::fopen(argv[1], "rb");
    if (!f) return 2;
    int64_t h[9];
    if (!read_all(f, h, sizeof h)) return 2;
    const int T = (int)h[0], k = (int)h[1], H = (int)h[2], I = (int)h[3], wdt = (int)h[4], nh = (int)h[5];
    const int64_t E = h[6], eb = h[7], reps = h[8];
    if (T < 1 || k < 1 || T * k > 1024 || nh < 1 || nh > T * k || reps < 1) return 2;
    std::vector<int32_t> ids(nh), rw((size_t)T * k);
    const size_t xb = (size_t)T * H * (wdt == 0 ? 4 : 2);
    std::vector<uint8_t> x(xb), bank((size_t)(E * eb));
    if (!read_all(f, ids.data(), 4 * ids.size()) || !read_all(f, rw.data(), 4 * rw.size()) ||
        !read_all(f, x.data(), xb) || !read_all(f, bank.data(), bank.size()))
        return 2;
    std::fclose(f);
    for (int i = 0; i < nh; ++i)
        if (ids[i] < 0 || ids[i] >= E) return 2;

    ec::HostJob j{};
    for (int i = 0; i < nh; ++i) j.expert_base[i] = bank.data() + (size_t)ids[i] * eb;
    j.n_experts = nh;
    j.rewritten = rw.data();
    j.T = T; j.k = k; j.H = H; j.I = I; j.wdtype = wdt;
    j.x = x.data();
    std::vector<float> act((size_t)T * k * I), first;
    j.act = act.data();
    const size_t ny = (size_t)T * H * k;
    std::vector<float> y(ny);
    const uint32_t sentinel = 0x7fc0beefu;
    ec::HostPool* pool = ec::host_pool_create(std::atoi(argv[3]));
    int rc = 0;
    for (int64_t r = 0; r < reps && rc == 0; ++r) {
        for (size_t i = 0; i < ny; ++i) std::memcpy(&y[i], &sentinel, 4);
        j.y = y.data();
        ec::host_pool_run(pool, j);
        for (int t = 0; t < T && rc == 0; ++t)
            for (int p = 0; p < k && rc == 0; ++p)
                if (rw[(size_t)t * k + p] >= 0)
                    for (int hh = 0; hh < H; ++hh) {
                        uint32_t u;
                        std::memcpy(&u, &y[((size_t)t * H + hh) * k + p], 4);
                        if (u != sentinel) { rc = 4; break; }
                    }
        if (r == 0) first = y;
        else if (std::memcmp(first.data(), y.data(), 4 * ny) != 0) rc = 3;
    }
    ec::host_pool_destroy(pool);
    if (rc) return rc;
    FILE* o = std::fopen(argv[2], "wb");
    if (!o || std::fwrite(y.data(), 4, ny, o) != ny) return 2;
    std::fclose(o);
    return 0;
}
