// Expert-bank files: the host pool stored in its final in-memory layout, read
// back with parallel direct I/O.
//
// FreeToken edge-MoE write-up, "Implementation notes": expert weights are kept
// in one "expert bank" layout (layer x expert as the leading dimensions) and
// written ahead of time in the runtime's layout, so loading skips tensor
// discovery and repacking and reads aligned blocks with parallel direct I/O;
// "Elastic edge resource management": loading straight into the final host
// layout keeps the cold start short.
//
// File format (little endian): a 4096-byte header, then the bank bytes.
//   0   char[8]  "ECBANK01"
//   8   u32      header version (1)
//   12  i32[6]   ec_shape: layers, experts, top_k, hidden, inter, wdtype
//   36  i32      pool layers P held by the file
//   40  u64      expert_bytes
//   48  u64      bank bytes (P * experts * expert_bytes)
//   56  u64      FNV-1a 64 of bytes 0..55
// The bank starts at byte 4096 and the file is padded to a multiple of 4096.
#include <fcntl.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <chrono>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "bank_io.h"

namespace ec {

namespace {

constexpr uint64_t kHeader = 4096, kAlign = 4096, kChunk = 32ull << 20;
constexpr char kMagic[8] = {'E', 'C', 'B', 'A', 'N', 'K', '0', '1'};

uint64_t fnv1a(const uint8_t* p, size_t n) {
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < n; ++i) h = (h ^ p[i]) * 1099511628211ull;
    return h;
}

void make_header(uint8_t* h, const int32_t shape[6], int32_t P, uint64_t expert_bytes, uint64_t bank_bytes) {
    std::memset(h, 0, kHeader);
    std::memcpy(h, kMagic, 8);
    const uint32_t ver = 1;
    std::memcpy(h + 8, &ver, 4);
    std::memcpy(h + 12, shape, 24);
    std::memcpy(h + 36, &P, 4);
    std::memcpy(h + 40, &expert_bytes, 8);
    std::memcpy(h + 48, &bank_bytes, 8);
    const uint64_t c = fnv1a(h, 56);
    std::memcpy(h + 56, &c, 8);
}

// pread until n bytes are read (or EOF / error)
bool read_full(int fd, uint8_t* dst, uint64_t n, uint64_t off) {
    while (n) {
        const ssize_t r = pread(fd, dst, n > (1ull << 30) ? (1ull << 30) : n, (off_t)off);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        dst += r; n -= (uint64_t)r; off += (uint64_t)r;
    }
    return true;
}

bool write_full(int fd, const uint8_t* src, uint64_t n, uint64_t off) {
    while (n) {
        const ssize_t r = pwrite(fd, src, n > (1ull << 30) ? (1ull << 30) : n, (off_t)off);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        src += r; n -= (uint64_t)r; off += (uint64_t)r;
    }
    return true;
}

} // namespace

int bank_write(const char* path, const int32_t shape[6], int32_t P, uint64_t expert_bytes, const void* bank,
               uint64_t bytes, std::string* err) {
    const int fd = open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (fd < 0) { *err = std::string("open for writing failed: ") + std::strerror(errno); return -1; }
    std::vector<uint8_t> h(kHeader);
    make_header(h.data(), shape, P, expert_bytes, bytes);
    bool ok = write_full(fd, h.data(), kHeader, 0) && write_full(fd, (const uint8_t*)bank, bytes, kHeader);
    const uint64_t end = kHeader + bytes, padded = (end + kAlign - 1) / kAlign * kAlign;
    if (ok && padded > end) {
        std::vector<uint8_t> z(padded - end, 0);
        ok = write_full(fd, z.data(), z.size(), end);
    }
    if (ok && fsync(fd) != 0) ok = false;
    if (close(fd) != 0) ok = false;
    if (!ok) *err = std::string("write failed: ") + std::strerror(errno);
    return ok ? 0 : -1;
}

int bank_read(const char* path, const int32_t shape[6], int32_t P, uint64_t expert_bytes, void* dst, uint64_t bytes,
              int threads, int* direct_used, double* seconds, std::string* err) {
    const auto t0 = std::chrono::steady_clock::now();
    // header through the page cache (one block), then the bank
    int fd = open(path, O_RDONLY);
    if (fd < 0) { *err = std::string("open failed: ") + std::strerror(errno); return -1; }
    std::vector<uint8_t> h(kHeader), want(kHeader);
    if (!read_full(fd, h.data(), kHeader, 0)) { close(fd); *err = "file shorter than its header"; return -1; }
    close(fd);
    make_header(want.data(), shape, P, expert_bytes, bytes);
    if (std::memcmp(h.data(), kMagic, 8) != 0) { *err = "not an expert-bank file"; return -2; }
    if (std::memcmp(h.data(), want.data(), 64) != 0) { *err = "bank file holds another shape, layer count or size"; return -2; }

    // Direct I/O needs aligned destinations, offsets and lengths. The bank is read in
    // whole 4096-byte blocks: straight into dst when the kernel can pin dst's pages for
    // the transfer (checked on the first block), else into per-reader aligned bounce
    // buffers copied to dst (memory handed out by a GPU driver may refuse direct
    // transfers); without O_DIRECT support, or for an unaligned dst, through the page
    // cache. The tail below 4096 bytes is always read buffered.
    enum Mode { kBuffered = 0, kDirect = 1, kBounce = 2 };
    int dfd = open(path, O_RDONLY | O_DIRECT);
    Mode mode = dfd >= 0 ? kDirect : kBuffered;
    if (mode == kDirect && (((uintptr_t)dst % kAlign) != 0 || bytes < kAlign ||
                            !read_full(dfd, (uint8_t*)dst, kAlign, kHeader)))
        mode = kBounce;
    if (mode == kBuffered) dfd = open(path, O_RDONLY);
    if (dfd < 0) { *err = std::string("open failed: ") + std::strerror(errno); return -1; }
    const uint64_t whole = mode == kBuffered ? bytes : bytes / kAlign * kAlign;
    const uint64_t nchunks = (whole + kChunk - 1) / kChunk;
    std::atomic<uint64_t> next{0};
    std::atomic<bool> failed{false};
    auto worker = [&] {
        uint8_t* bounce = nullptr;
        if (mode == kBounce && posix_memalign((void**)&bounce, kAlign, kChunk) != 0) { failed = true; return; }
        for (uint64_t c; (c = next.fetch_add(1)) < nchunks && !failed.load();) {
            const uint64_t off = c * kChunk, n = std::min(kChunk, whole - off);
            uint8_t* to = (uint8_t*)dst + off;
            if (mode == kBounce) {
                if (!read_full(dfd, bounce, n, kHeader + off)) failed = true;
                else std::memcpy(to, bounce, n);
            } else if (!read_full(dfd, to, n, kHeader + off)) {
                failed = true;
            }
        }
        std::free(bounce);
    };
    const int nt = std::max(1, std::min(threads, 64));
    std::vector<std::thread> pool;
    for (int i = 1; i < nt; ++i) pool.emplace_back(worker);
    worker();
    for (auto& t : pool) t.join();
    close(dfd);
    if (!failed && whole < bytes) {
        int bfd = open(path, O_RDONLY);
        if (bfd < 0 || !read_full(bfd, (uint8_t*)dst + whole, bytes - whole, kHeader + whole)) failed = true;
        if (bfd >= 0) close(bfd);
    }
    if (failed) { *err = "read failed or file truncated"; return -1; }
    if (direct_used) *direct_used = (int)mode;
    if (seconds) *seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    return 0;
}

} // namespace ec
