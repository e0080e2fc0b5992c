// Stored stack on disk: packed planes of many matrices, plane-major, so that
// a read at depth d is one contiguous prefix of the plane sections plus the
// scales section ([FoQLens] "Progress": one stored copy read at 2, 4, 6 or 8
// bits without repacking).  Host code only: POSIX file I/O, pinned staging
// buffers and asynchronous copies on the caller's stream.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cstring>
#include <vector>

#include "qam_common.h"

static_assert(sizeof(qam_stack_header) == 128, "stack header is 128 bytes");
static_assert(sizeof(qam_stack_entry) == 64, "stack entry is 64 bytes");
static_assert(offsetof(qam_stack_header, data_offset) == 40, "stack header field offsets");

namespace qam {
namespace {

constexpr char kMagic[8] = {'Q', 'A', 'M', 'S', 'T', 'A', 'C', 'K'};
constexpr uint8_t kLadder[5] = {0, 2, 4, 6, 8};
constexpr size_t kStageBytes = 32u << 20;   // one pinned staging buffer

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Offsets of a stack with these shapes, filled into a header and entries.
void lay_out(const int64_t* N, const int64_t* K, int n, qam_stack_header& h, std::vector<qam_stack_entry>& e) {
    std::memset(&h, 0, sizeof(h));
    std::memcpy(h.magic, kMagic, 8);
    h.version = QAM_STACK_VERSION;
    h.n_matrices = (uint32_t)n;
    h.n_rungs = 5;
    std::memcpy(h.ladder_bits, kLadder, 5);
    h.rows_per_block = QAM_ROWS_PER_BLOCK;
    e.assign((size_t)n, qam_stack_entry{});
    uint64_t plane = 0, scales = 0;
    for (int m = 0; m < n; ++m) {
        e[m].N = N[m];
        e[m].K = K[m];
        e[m].plane_offset = plane;
        e[m].scales_offset = scales;
        plane += (uint64_t)N[m] * (uint64_t)K[m] / 4;
        scales += 4 * (uint64_t)N[m];
    }
    h.data_offset = round_up(sizeof(qam_stack_header) + sizeof(qam_stack_entry) * (uint64_t)n, QAM_STACK_ALIGN);
    h.plane_section_bytes = plane;
    h.scales_offset = h.data_offset + 4 * plane;
    h.scales_bytes = scales;
    h.file_bytes = h.scales_offset + scales;
}

bool good_shape(int64_t N, int64_t K) {
    return N > 0 && K > 0 && N % QAM_ROWS_PER_BLOCK == 0 && K % 64 == 0 && K <= QAM_MAX_K &&
           N / QAM_ROWS_PER_BLOCK <= QAM_MAX_BLOCKS;
}

// RAII holders for a file descriptor and pinned host buffers.
struct Fd {
    int fd = -1;
    ~Fd() {
        if (fd >= 0) close(fd);
    }
};

struct Pinned {
    void* p[2] = {nullptr, nullptr};
    hipEvent_t ev[2] = {nullptr, nullptr};
    hipStream_t s = nullptr;
    ~Pinned() {
        (void)hipStreamSynchronize(s);   // no copy may still use a buffer freed here
        for (int i = 0; i < 2; ++i) {
            if (ev[i]) (void)hipEventDestroy(ev[i]);
            if (p[i]) (void)hipHostFree(p[i]);
        }
    }
    int init(size_t bytes, hipStream_t stream) {
        s = stream;
        for (int i = 0; i < 2; ++i) {
            QAM_HIP_CHECK(hipHostMalloc(&p[i], bytes, hipHostMallocDefault));
            QAM_HIP_CHECK(hipEventCreateWithFlags(&ev[i], hipEventDisableTiming));
        }
        return QAM_OK;
    }
};

bool write_all(int fd, const void* buf, size_t n, uint64_t off) {
    const char* c = static_cast<const char*>(buf);
    while (n) {
        const ssize_t w = pwrite(fd, c, n, (off_t)off);
        if (w < 0 && errno == EINTR) continue;
        if (w <= 0) return false;
        c += w, n -= (size_t)w, off += (uint64_t)w;
    }
    return true;
}

bool read_all(int fd, void* buf, size_t n, uint64_t off) {
    char* c = static_cast<char*>(buf);
    while (n) {
        const ssize_t r = pread(fd, c, n, (off_t)off);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        c += r, n -= (size_t)r, off += (uint64_t)r;
    }
    return true;
}

// One piece of a transfer: `bytes` at file offset `file` <-> device address `dev`.
struct Piece {
    uint64_t file;
    char* dev;
    size_t bytes;
};

// Reads the header and table of an open stack file and checks them.
int load_table(int fd, const char* path, qam_stack_header& h, std::vector<qam_stack_entry>& e) {
    struct stat st;
    if (fstat(fd, &st) != 0) QAM_FAIL(QAM_ERR_IO, "stack: cannot stat %s", path);
    if ((uint64_t)st.st_size < sizeof(h) || !read_all(fd, &h, sizeof(h), 0))
        QAM_FAIL(QAM_ERR_IO, "stack: %s is too short for a header", path);
    if (std::memcmp(h.magic, kMagic, 8) != 0) QAM_FAIL(QAM_ERR_IO, "stack: %s has no QAMSTACK magic", path);
    if (h.version != QAM_STACK_VERSION)
        QAM_FAIL(QAM_ERR_IO, "stack: %s has version %u, expected %d", path, h.version, QAM_STACK_VERSION);
    if (h.n_matrices < 1 || h.n_matrices > QAM_STACK_MAX_MATRICES)
        QAM_FAIL(QAM_ERR_IO, "stack: %s holds %u matrices", path, h.n_matrices);
    if (h.n_rungs != 5 || std::memcmp(h.ladder_bits, kLadder, 5) != 0 || h.rows_per_block != QAM_ROWS_PER_BLOCK)
        QAM_FAIL(QAM_ERR_IO, "stack: %s is not a {0,2,4,6,8} stack of 64-row blocks", path);
    for (int i = 5; i < 16; ++i)
        if (h.ladder_bits[i]) QAM_FAIL(QAM_ERR_IO, "stack: %s has ladder bytes past the fifth rung", path);
    for (uint8_t r : h.reserved)
        if (r) QAM_FAIL(QAM_ERR_IO, "stack: %s has nonzero reserved header bytes", path);
    const size_t tbytes = sizeof(qam_stack_entry) * (size_t)h.n_matrices;
    if ((uint64_t)st.st_size < sizeof(h) + tbytes) QAM_FAIL(QAM_ERR_IO, "stack: %s is too short for its table", path);
    std::vector<qam_stack_entry> got((size_t)h.n_matrices);
    if (!read_all(fd, got.data(), tbytes, sizeof(h))) QAM_FAIL(QAM_ERR_IO, "stack: cannot read the table of %s", path);
    std::vector<int64_t> N(got.size()), K(got.size());
    for (size_t m = 0; m < got.size(); ++m) {
        if (!good_shape(got[m].N, got[m].K))
            QAM_FAIL(QAM_ERR_IO, "stack: %s entry %zu has a bad shape %lld x %lld", path, m, (long long)got[m].N,
                     (long long)got[m].K);
        N[m] = got[m].N, K[m] = got[m].K;
    }
    qam_stack_header want;
    lay_out(N.data(), K.data(), (int)got.size(), want, e);
    if (h.data_offset != want.data_offset || h.plane_section_bytes != want.plane_section_bytes ||
        h.scales_offset != want.scales_offset || h.scales_bytes != want.scales_bytes ||
        h.file_bytes != want.file_bytes)
        QAM_FAIL(QAM_ERR_IO, "stack: %s has offsets that do not follow from its shapes", path);
    for (size_t m = 0; m < got.size(); ++m) {
        if (got[m].plane_offset != e[m].plane_offset || got[m].scales_offset != e[m].scales_offset)
            QAM_FAIL(QAM_ERR_IO, "stack: %s entry %zu has offsets that do not follow from the shapes", path, m);
        std::memcpy(e[m].name, got[m].name, QAM_STACK_NAME_BYTES);
    }
    if ((uint64_t)st.st_size != h.file_bytes)
        QAM_FAIL(QAM_ERR_IO, "stack: %s is %lld bytes, its header says %llu", path, (long long)st.st_size,
                 (unsigned long long)h.file_bytes);
    return QAM_OK;
}

}  // namespace
}  // namespace qam

using namespace qam;

extern "C" int qam_stack_write(const char* path, const qam_packed* mats, const char* const* names, int n_matrices,
                               hipStream_t s) {
    clear_error();
    if (!path || !mats) QAM_FAIL(QAM_ERR_NULL, "stack_write: null pointer");
    if (n_matrices < 1 || n_matrices > QAM_STACK_MAX_MATRICES)
        QAM_FAIL(QAM_ERR_ARG, "stack_write: n_matrices=%d outside [1, %d]", n_matrices, QAM_STACK_MAX_MATRICES);
    std::vector<int64_t> N((size_t)n_matrices), K((size_t)n_matrices);
    for (int m = 0; m < n_matrices; ++m) {
        const qam_packed& w = mats[m];
        if (!good_shape(w.N, w.K) || w.n_blocks != w.N / QAM_ROWS_PER_BLOCK)
            QAM_FAIL(QAM_ERR_SHAPE, "stack_write: matrix %d has a bad shape", m);
        if (!w.planes || w.scales != reinterpret_cast<float*>(static_cast<char*>(w.planes) + w.N * w.K))
            QAM_FAIL(QAM_ERR_ARG, "stack_write: matrix %d is not a packed descriptor", m);
        if (names && names[m] && std::strlen(names[m]) >= QAM_STACK_NAME_BYTES)
            QAM_FAIL(QAM_ERR_ARG, "stack_write: name of matrix %d is longer than %d characters", m,
                     QAM_STACK_NAME_BYTES - 1);
        N[m] = w.N, K[m] = w.K;
    }
    qam_stack_header h;
    std::vector<qam_stack_entry> e;
    lay_out(N.data(), K.data(), n_matrices, h, e);
    for (int m = 0; m < n_matrices; ++m)
        if (names && names[m]) std::strncpy(e[m].name, names[m], QAM_STACK_NAME_BYTES - 1);

    // transfer list in file order
    std::vector<Piece> pieces;
    for (int p = 0; p < 4; ++p)
        for (int m = 0; m < n_matrices; ++m) {
            const uint64_t pb = (uint64_t)N[m] * (uint64_t)K[m] / 4;
            pieces.push_back({h.data_offset + p * h.plane_section_bytes + e[m].plane_offset,
                              static_cast<char*>(mats[m].planes) + p * pb, (size_t)pb});
        }
    for (int m = 0; m < n_matrices; ++m)
        pieces.push_back({h.scales_offset + e[m].scales_offset, reinterpret_cast<char*>(mats[m].scales),
                          (size_t)(4 * N[m])});

    QAM_HIP_CHECK(hipStreamSynchronize(s));
    Fd f;
    f.fd = open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (f.fd < 0) QAM_FAIL(QAM_ERR_IO, "stack_write: cannot create %s: %s", path, std::strerror(errno));
    std::vector<char> head((size_t)h.data_offset, 0);
    std::memcpy(head.data(), &h, sizeof(h));
    std::memcpy(head.data() + sizeof(h), e.data(), sizeof(qam_stack_entry) * e.size());
    if (!write_all(f.fd, head.data(), head.size(), 0)) QAM_FAIL(QAM_ERR_IO, "stack_write: cannot write %s", path);

    // device -> pinned buffer k (async), then write it out while buffer k^1 fills
    Pinned st;
    if (int rc = st.init(kStageBytes, s)) return rc;
    struct Batch {
        uint64_t file = 0;
        size_t bytes = 0;
    };
    Batch pending[2];
    int k = 0;
    size_t fill = 0;
    uint64_t batch_file = 0;
    auto flush = [&](int b) -> bool {
        if (!pending[b].bytes) return true;
        if (hipEventSynchronize(st.ev[b]) != hipSuccess) return false;
        const bool ok = write_all(f.fd, st.p[b], pending[b].bytes, pending[b].file);
        pending[b].bytes = 0;
        return ok;
    };
    for (const Piece& pc : pieces) {
        size_t done = 0;
        while (done < pc.bytes) {
            if (fill == 0) batch_file = pc.file + done;
            const bool contiguous = batch_file + fill == pc.file + done;
            if (!contiguous || fill == kStageBytes) {   // close buffer k, switch
                QAM_HIP_CHECK(hipEventRecord(st.ev[k], s));
                pending[k] = {batch_file, fill};
                k ^= 1;
                if (!flush(k)) QAM_FAIL(QAM_ERR_IO, "stack_write: cannot write %s", path);
                fill = 0;
                batch_file = pc.file + done;
            }
            const size_t n = std::min(pc.bytes - done, kStageBytes - fill);
            QAM_HIP_CHECK(hipMemcpyAsync(static_cast<char*>(st.p[k]) + fill, pc.dev + done, n,
                                         hipMemcpyDeviceToHost, s));
            fill += n, done += n;
        }
    }
    if (fill) {
        QAM_HIP_CHECK(hipEventRecord(st.ev[k], s));
        pending[k] = {batch_file, fill};
    }
    if (!flush(k ^ 1) || !flush(k)) QAM_FAIL(QAM_ERR_IO, "stack_write: cannot write %s", path);
    if (fsync(f.fd) != 0) QAM_FAIL(QAM_ERR_IO, "stack_write: cannot sync %s: %s", path, std::strerror(errno));
    set_variant("stack_write");
    return QAM_OK;
}

extern "C" int qam_stack_info(const char* path, qam_stack_header* hdr_out, qam_stack_entry* entries_out,
                              int max_entries) {
    clear_error();
    if (!path || !hdr_out) QAM_FAIL(QAM_ERR_NULL, "stack_info: null pointer");
    if (max_entries < 0 || (max_entries > 0 && !entries_out))
        QAM_FAIL(QAM_ERR_ARG, "stack_info: entries_out must hold max_entries >= 0 entries");
    Fd f;
    f.fd = open(path, O_RDONLY);
    if (f.fd < 0) QAM_FAIL(QAM_ERR_IO, "stack_info: cannot open %s: %s", path, std::strerror(errno));
    qam_stack_header h;
    std::vector<qam_stack_entry> e;
    if (int rc = load_table(f.fd, path, h, e)) return rc;
    *hdr_out = h;
    const int n = std::min<int>(max_entries, (int)e.size());
    for (int m = 0; m < n; ++m) entries_out[m] = e[m];
    return QAM_OK;
}

extern "C" int qam_stack_read(const char* path, int slices, int first, int count, const qam_packed* dst,
                              hipStream_t s, uint64_t* bytes_read) {
    clear_error();
    if (!path || !dst) QAM_FAIL(QAM_ERR_NULL, "stack_read: null pointer");
    if (slices < 1 || slices > 4) QAM_FAIL(QAM_ERR_ARG, "stack_read: slices=%d outside [1, 4]", slices);
    Fd f;
    f.fd = open(path, O_RDONLY);
    if (f.fd < 0) QAM_FAIL(QAM_ERR_IO, "stack_read: cannot open %s: %s", path, std::strerror(errno));
    qam_stack_header h;
    std::vector<qam_stack_entry> e;
    if (int rc = load_table(f.fd, path, h, e)) return rc;
    if (first < 0 || count < 1 || (int64_t)first + count > (int64_t)e.size())
        QAM_FAIL(QAM_ERR_ARG, "stack_read: matrices [%d, %lld) outside the file's %zu", first,
                 (long long)first + count, e.size());
    for (int i = 0; i < count; ++i) {
        const qam_packed& w = dst[i];
        const qam_stack_entry& en = e[(size_t)first + i];
        if (w.N != en.N || w.K != en.K || w.n_blocks != en.N / QAM_ROWS_PER_BLOCK)
            QAM_FAIL(QAM_ERR_SHAPE, "stack_read: destination %d is %lld x %lld, the file holds %lld x %lld", i,
                     (long long)w.N, (long long)w.K, (long long)en.N, (long long)en.K);
        if (!w.planes || w.scales != reinterpret_cast<float*>(static_cast<char*>(w.planes) + w.N * w.K))
            QAM_FAIL(QAM_ERR_ARG, "stack_read: destination %d is not a packed descriptor", i);
    }
    std::vector<Piece> pieces;
    uint64_t total = 0;
    for (int p = 0; p < slices; ++p)
        for (int i = 0; i < count; ++i) {
            const qam_stack_entry& en = e[(size_t)first + i];
            const uint64_t pb = (uint64_t)en.N * (uint64_t)en.K / 4;
            pieces.push_back({h.data_offset + p * h.plane_section_bytes + en.plane_offset,
                              static_cast<char*>(dst[i].planes) + p * pb, (size_t)pb});
            total += pb;
        }
    for (int i = 0; i < count; ++i) {
        const qam_stack_entry& en = e[(size_t)first + i];
        pieces.push_back({h.scales_offset + en.scales_offset, reinterpret_cast<char*>(dst[i].scales),
                          (size_t)(4 * en.N)});
        total += 4 * (uint64_t)en.N;
    }
    // planes below the read depth read as zero digits
    for (int i = 0; i < count && slices < 4; ++i) {
        const uint64_t pb = (uint64_t)dst[i].N * (uint64_t)dst[i].K / 4;
        QAM_HIP_CHECK(hipMemsetAsync(static_cast<char*>(dst[i].planes) + slices * pb, 0, (4 - slices) * pb, s));
    }

    // file -> pinned buffer k, then buffer k -> device (async) while buffer k^1 fills
    Pinned st;
    if (int rc = st.init(kStageBytes, s)) return rc;
    bool used[2] = {false, false};
    int k = 0;
    size_t fill = 0;
    std::vector<Piece> staged;   // pieces of the buffer being filled: dev, bytes, offset in buffer
    auto issue = [&]() -> int {
        for (const Piece& q : staged)
            QAM_HIP_CHECK(hipMemcpyAsync(q.dev, static_cast<char*>(st.p[k]) + q.file, q.bytes,
                                         hipMemcpyHostToDevice, s));
        QAM_HIP_CHECK(hipEventRecord(st.ev[k], s));
        used[k] = true;
        staged.clear();
        fill = 0;
        k ^= 1;
        if (used[k]) QAM_HIP_CHECK(hipEventSynchronize(st.ev[k]));   // its copies are done: reuse it
        return QAM_OK;
    };
    for (const Piece& pc : pieces) {
        size_t done = 0;
        while (done < pc.bytes) {
            const size_t n = std::min(pc.bytes - done, kStageBytes - fill);
            if (!read_all(f.fd, static_cast<char*>(st.p[k]) + fill, n, pc.file + done))
                QAM_FAIL(QAM_ERR_IO, "stack_read: cannot read %s", path);
            staged.push_back({(uint64_t)fill, pc.dev + done, n});
            fill += n, done += n;
            if (fill == kStageBytes)
                if (int rc = issue()) return rc;
        }
    }
    if (fill)
        if (int rc = issue()) return rc;
    QAM_HIP_CHECK(hipStreamSynchronize(s));
    if (bytes_read) *bytes_read = total;
    char v[96];
    snprintf(v, sizeof(v), "stack_read slices=%d matrices=%d", slices, count);
    set_variant(v);
    return QAM_OK;
}
