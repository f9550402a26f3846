// Persisted packed pool: the encoded layer blocks of a stack in one file, so a
// later process reads them straight back (into pinned host memory for
// streaming, or through it into device memory) instead of encoding the
// weights again.
//
// File layout (little-endian):
//   0   char[8]   "WOQPOOL1"
//   8   uint32    version (1)
//   12  uint32    n_blocks
//   16  uint64    meta_bytes
//   24  uint64    header checksum (of the table and the meta bytes)
//   32  n_blocks x {uint64 offset, uint64 bytes, uint64 checksum}
//   ..  meta bytes (opaque to the library)
//   blocks, each at a 4096-byte aligned offset
// A block's checksum hashes the 64-bit hashes of its 1 MiB chunks (each a
// 64-bit FNV-1a over little-endian 8-byte words, the tail zero-padded), so
// chunks are hashed in parallel and the value does not depend on the thread
// count.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <cstring>
#include <vector>

#include "woq_internal.h"

namespace {

constexpr char MAGIC[8] = {'W', 'O', 'Q', 'P', 'O', 'O', 'L', '1'};
constexpr uint32_t VERSION = 1;
constexpr int64_t CHUNK = 1 << 20;
constexpr int64_t ALIGN = 4096;
constexpr uint64_t FNV_OFFSET = 0xcbf29ce484222325ull, FNV_PRIME = 0x100000001b3ull;

struct Entry {
    uint64_t offset, bytes, checksum;
};

uint64_t fnv_words(const uint8_t* p, int64_t n, uint64_t h = FNV_OFFSET) {
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
        uint64_t w;
        std::memcpy(&w, p + i, 8);
        h = (h ^ w) * FNV_PRIME;
    }
    if (i < n) {
        uint64_t w = 0;
        std::memcpy(&w, p + i, (size_t)(n - i));
        h = (h ^ w) * FNV_PRIME;
    }
    return h;
}

uint64_t combine(const std::vector<uint64_t>& chunk_hashes) {
    return fnv_words(reinterpret_cast<const uint8_t*>(chunk_hashes.data()), (int64_t)(8 * chunk_hashes.size()));
}

uint64_t block_checksum(const uint8_t* p, int64_t n) {
    const int64_t nc = woq::ceil_div(n, CHUNK);
    std::vector<uint64_t> hs((size_t)nc, 0);
    woq::parallel_for(nc, [&](int64_t lo, int64_t hi) {
        for (int64_t c = lo; c < hi; ++c) hs[(size_t)c] = fnv_words(p + c * CHUNK, std::min(CHUNK, n - c * CHUNK));
    });
    return combine(hs);
}

bool full_pwrite(int fd, const void* buf, int64_t n, int64_t off) {
    const uint8_t* p = (const uint8_t*)buf;
    while (n > 0) {
        ssize_t w = pwrite(fd, p, (size_t)std::min<int64_t>(n, 1 << 30), off);
        if (w < 0 && errno == EINTR) continue;
        if (w <= 0) return false;
        p += w;
        n -= w;
        off += w;
    }
    return true;
}

// 1 on success, 0 on a short read (end of file), -1 on an error
int full_pread(int fd, void* buf, int64_t n, int64_t off) {
    uint8_t* p = (uint8_t*)buf;
    while (n > 0) {
        ssize_t r = pread(fd, p, (size_t)std::min<int64_t>(n, 1 << 30), off);
        if (r < 0 && errno == EINTR) continue;
        if (r < 0) return -1;
        if (r == 0) return 0;
        p += r;
        n -= r;
        off += r;
    }
    return 1;
}

struct Header {
    uint32_t n_blocks = 0;
    uint64_t meta_bytes = 0;
    std::vector<Entry> table;
    std::vector<uint8_t> meta;
};

uint64_t header_checksum(const std::vector<Entry>& table, const std::vector<uint8_t>& meta) {
    uint64_t h = fnv_words(reinterpret_cast<const uint8_t*>(table.data()), (int64_t)(sizeof(Entry) * table.size()));
    return fnv_words(meta.data(), (int64_t)meta.size(), h);
}

// Read and check the header of an open pool file.
int read_header(int fd, Header& h) {
    uint8_t fixed[32];
    int r = full_pread(fd, fixed, 32, 0);
    if (r < 0) return WOQ_EIO;
    if (r == 0 || std::memcmp(fixed, MAGIC, 8) != 0) return WOQ_EFORMAT;
    uint32_t version;
    uint64_t stored;
    std::memcpy(&version, fixed + 8, 4);
    std::memcpy(&h.n_blocks, fixed + 12, 4);
    std::memcpy(&h.meta_bytes, fixed + 16, 8);
    std::memcpy(&stored, fixed + 24, 8);
    struct stat sb;
    if (fstat(fd, &sb) != 0) return WOQ_EIO;
    const uint64_t fsize = (uint64_t)sb.st_size;
    if (version != VERSION || h.n_blocks > (1u << 20) || h.meta_bytes > fsize ||
        32 + sizeof(Entry) * (uint64_t)h.n_blocks + h.meta_bytes > fsize)
        return WOQ_EFORMAT;
    h.table.resize(h.n_blocks);
    h.meta.resize((size_t)h.meta_bytes);
    if (h.n_blocks && full_pread(fd, h.table.data(), (int64_t)(sizeof(Entry) * h.n_blocks), 32) != 1) return WOQ_EFORMAT;
    if (h.meta_bytes &&
        full_pread(fd, h.meta.data(), (int64_t)h.meta_bytes, 32 + (int64_t)(sizeof(Entry) * h.n_blocks)) != 1)
        return WOQ_EFORMAT;
    if (header_checksum(h.table, h.meta) != stored) return WOQ_EFORMAT;
    for (const Entry& e : h.table)
        if (e.offset % ALIGN || e.offset > fsize || e.bytes > fsize - e.offset) return WOQ_EFORMAT;
    return WOQ_OK;
}

struct Fd {
    int fd = -1;
    ~Fd() {
        if (fd >= 0) close(fd);
    }
};

}  // namespace

extern "C" {

int woq_pool_save(const char* path, const void* meta, int64_t meta_bytes, const void* const* blocks,
                  const int64_t* block_bytes, int32_t n_blocks) {
    if (!path || meta_bytes < 0 || (meta_bytes > 0 && !meta) || n_blocks < 0 || (n_blocks > 0 && (!blocks || !block_bytes)))
        return WOQ_EINVAL;
    for (int i = 0; i < n_blocks; ++i)
        if (block_bytes[i] < 0 || (block_bytes[i] > 0 && !blocks[i])) return WOQ_EINVAL;
    std::vector<Entry> table((size_t)n_blocks);
    int64_t off = woq::round_up(32 + (int64_t)sizeof(Entry) * n_blocks + meta_bytes, ALIGN);
    for (int i = 0; i < n_blocks; ++i) {
        table[i].offset = (uint64_t)off;
        table[i].bytes = (uint64_t)block_bytes[i];
        table[i].checksum = block_checksum((const uint8_t*)blocks[i], block_bytes[i]);
        off = woq::round_up(off + block_bytes[i], ALIGN);
    }
    std::vector<uint8_t> m((const uint8_t*)meta, (const uint8_t*)meta + meta_bytes);
    uint8_t fixed[32];
    std::memcpy(fixed, MAGIC, 8);
    const uint32_t nb = (uint32_t)n_blocks;
    const uint64_t mb = (uint64_t)meta_bytes, hc = header_checksum(table, m);
    std::memcpy(fixed + 8, &VERSION, 4);
    std::memcpy(fixed + 12, &nb, 4);
    std::memcpy(fixed + 16, &mb, 8);
    std::memcpy(fixed + 24, &hc, 8);
    Fd f;
    f.fd = open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (f.fd < 0) return WOQ_EIO;
    bool ok = full_pwrite(f.fd, fixed, 32, 0) &&
              (n_blocks == 0 || full_pwrite(f.fd, table.data(), (int64_t)sizeof(Entry) * n_blocks, 32)) &&
              (meta_bytes == 0 || full_pwrite(f.fd, m.data(), meta_bytes, 32 + (int64_t)sizeof(Entry) * n_blocks));
    for (int i = 0; i < n_blocks && ok; ++i) {
        const uint8_t* src = (const uint8_t*)blocks[i];
        const int64_t base = (int64_t)table[i].offset, n = block_bytes[i];
        std::atomic<bool> good{true};
        woq::parallel_for(woq::ceil_div(n, CHUNK * 8), [&](int64_t lo, int64_t hi) {
            for (int64_t c = lo; c < hi; ++c) {
                const int64_t o = c * CHUNK * 8, len = std::min(CHUNK * 8, n - o);
                if (!full_pwrite(f.fd, src + o, len, base + o)) good = false;
            }
        });
        ok = good;
    }
    // the file ends at the last block's aligned end
    if (ok && ftruncate(f.fd, off) != 0) ok = false;
    if (ok && fsync(f.fd) != 0) ok = false;
    return ok ? WOQ_OK : WOQ_EIO;
}

int woq_pool_info(const char* path, int32_t* n_blocks, int64_t* meta_bytes, int64_t* block_bytes, int32_t max_blocks,
                  void* meta, int64_t meta_cap) {
    if (!path || !n_blocks || !meta_bytes || max_blocks < 0 || meta_cap < 0) return WOQ_EINVAL;
    Fd f;
    f.fd = open(path, O_RDONLY);
    if (f.fd < 0) return WOQ_EIO;
    Header h;
    int rc = read_header(f.fd, h);
    if (rc) return rc;
    *n_blocks = (int32_t)h.n_blocks;
    *meta_bytes = (int64_t)h.meta_bytes;
    if (block_bytes)
        for (uint32_t i = 0; i < h.n_blocks && (int32_t)i < max_blocks; ++i) block_bytes[i] = (int64_t)h.table[i].bytes;
    if (meta && h.meta_bytes) std::memcpy(meta, h.meta.data(), (size_t)std::min<int64_t>(meta_cap, h.meta_bytes));
    return WOQ_OK;
}

int woq_pool_read_block(const char* path, int32_t i, void* dst, int64_t dst_bytes) {
    if (!path || i < 0 || !dst || dst_bytes < 0) return WOQ_EINVAL;
    Fd f;
    f.fd = open(path, O_RDONLY);
    if (f.fd < 0) return WOQ_EIO;
    Header h;
    int rc = read_header(f.fd, h);
    if (rc) return rc;
    if ((uint32_t)i >= h.n_blocks) return WOQ_EINVAL;
    const Entry& e = h.table[(size_t)i];
    if ((int64_t)e.bytes > dst_bytes) return WOQ_EINVAL;
    const int64_t n = (int64_t)e.bytes;
    const int64_t nc = woq::ceil_div(n, CHUNK);
    std::vector<uint64_t> hs((size_t)nc, 0);
    std::atomic<int> bad{0};
    uint8_t* out = (uint8_t*)dst;
    woq::parallel_for(nc, [&](int64_t lo, int64_t hi) {
        // each worker reads its contiguous run of chunks with large reads,
        // then hashes them while they are in cache
        const int64_t o = lo * CHUNK, len = std::min(hi * CHUNK, n) - o;
        const int r = full_pread(f.fd, out + o, len, (int64_t)e.offset + o);
        if (r != 1) {
            bad = r < 0 ? WOQ_EIO : WOQ_EFORMAT;
            return;
        }
        for (int64_t c = lo; c < hi; ++c) hs[(size_t)c] = fnv_words(out + c * CHUNK, std::min(CHUNK, n - c * CHUNK));
    });
    if (bad) return bad;
    return combine(hs) == e.checksum ? WOQ_OK : WOQ_EFORMAT;
}

}  // extern "C"
