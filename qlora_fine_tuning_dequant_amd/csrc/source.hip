// Disk stream source. The frozen base may sit in CPU memory or on disk
// (rug.gal article, "En detalle"), and the tool's `stream_source: auto`
// setting takes RAM when the stack fits there and the NVMe disk otherwise
// (imasters article, "Como cabe um 8B em 4 GB"). Here the stack is one file, layer i's blob
// at offset i * stride (stride = the blob size rounded up to 4 KiB, zero
// padded), read with O_DIRECT where the file system allows it, so a read is a
// disk read and not a page-cache copy. A read is split into 8 MiB jobs served
// by 16 reader threads (a whole layer's requests in flight on the device)
// through per-thread bounce buffers; the
// streamer reads into one of two pinned staging buffers and copies that to a
// device slot, so disk, host link and compute form a three-stage pipeline.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "layer.h"
#include "source.h"

namespace qlx {

static std::string errstr(int e) { return std::string(std::strerror(e)); }

// A direct read cannot land in the runtime's pinned allocation (the kernel
// cannot pin those pages for the transfer: EFAULT), so with O_DIRECT each
// reader reads into its own aligned bounce buffer and copies from there; the
// copies of one layer's chunks run on the reader threads in parallel with the
// other chunks' reads.
static void reader(qlx_layer_file* f) {
    void* bounce = nullptr;
    if (f->direct && posix_memalign(&bounce, kFileAlign, kReadChunk) != 0) bounce = nullptr;
    std::unique_lock<std::mutex> lk(f->mu);
    for (;;) {
        f->cv_job.wait(lk, [&] { return f->stop || !f->jobs.empty(); });
        if (f->jobs.empty()) {  // stop requested and nothing left
            lk.unlock();
            std::free(bounce);
            return;
        }
        const qlx_layer_file::Job j = f->jobs.front();
        f->jobs.pop_front();
        lk.unlock();
        int err = (f->direct && !bounce) ? ENOMEM : 0;
        bool ended = false;
        uint64_t done = 0;
        char* buf = f->direct ? static_cast<char*>(bounce) : j.dst;
        while (!err && done < j.len) {
            const ssize_t r = pread(f->fd, buf + done, size_t(j.len - done), off_t(j.off + done));
            if (r < 0) {
                if (errno == EINTR) continue;
                err = errno;
                break;
            }
            if (r == 0) {
                ended = true;
                break;
            }
            done += uint64_t(r);
        }
        if (f->direct && !err) std::memcpy(j.dst, bounce, size_t(done));
        lk.lock();
        if (err && !f->io_errno) f->io_errno = err;
        if (ended) f->short_read = true;
        if (--f->pending == 0) f->cv_done.notify_all();
    }
}

void layer_file_read(qlx_layer_file* f, int layer, void* dst) {
    QLX_REQUIRE(layer >= 0 && layer < f->dims.n_layers, QLX_EINVAL, "layer index out of range");
    QLX_REQUIRE((reinterpret_cast<uintptr_t>(dst) % kFileAlign) == 0, QLX_EINVAL, "read buffer must be 4 KiB aligned");
    std::unique_lock<std::mutex> lk(f->mu);
    f->io_errno = 0;
    f->short_read = false;
    const uint64_t base = uint64_t(layer) * f->stride;
    for (uint64_t o = 0; o < f->stride; o += kReadChunk) {
        f->jobs.push_back({static_cast<char*>(dst) + o, base + o, std::min(kReadChunk, f->stride - o)});
        ++f->pending;
    }
    f->cv_job.notify_all();
    f->cv_done.wait(lk, [&] { return f->pending == 0; });
    QLX_REQUIRE(f->io_errno == 0, QLX_EIO,
                "reading layer " + std::to_string(layer) + " of " + f->path + ": " + errstr(f->io_errno));
    QLX_REQUIRE(!f->short_read, QLX_EIO, "reading layer " + std::to_string(layer) + " of " + f->path + ": file ends early");
}

static uint64_t stride_of(const qlx_dims& d, int form, uint64_t* blob_bytes) {
    uint64_t off[QLX_BLOB_NSEG];
    if (form == QLX_BLOB_WIRE) wire_layout(d, off, blob_bytes);
    else blob_layout(d, off, blob_bytes);
    return (*blob_bytes + kFileAlign - 1) / kFileAlign * kFileAlign;
}

static void close_file(qlx_layer_file* f) {
    {
        std::lock_guard<std::mutex> lk(f->mu);
        f->stop = true;
    }
    f->cv_job.notify_all();
    for (auto& t : f->workers) t.join();
    if (f->device >= 0) {
        (void)hipSetDevice(f->device);
        for (int k = 0; k < kStaging; ++k) {
            if (f->staging_free[k]) {
                (void)hipEventSynchronize(f->staging_free[k]);  // no copy still reads the buffer
                (void)hipEventDestroy(f->staging_free[k]);
            }
            if (f->staging[k]) (void)hipHostFree(f->staging[k]);
        }
    }
    if (f->fd >= 0) close(f->fd);
    delete f;
}

}  // namespace qlx

using namespace qlx;

extern "C" {

int qlx_layer_file_write(const char* path, const qlx_dims* d, const void* const* blobs, int flags) {
    return guarded([&] {
        REQ_PTR(path, "path");
        REQ_PTR(blobs, "blobs");
        validate_dims(d);
        QLX_REQUIRE((flags & ~QLX_FILE_WIRE) == 0, QLX_EINVAL, "layer-file write flags: 0 or QLX_FILE_WIRE");
        uint64_t blob_bytes = 0;
        const uint64_t stride = stride_of(*d, (flags & QLX_FILE_WIRE) ? QLX_BLOB_WIRE : QLX_BLOB_FULL, &blob_bytes);
        for (int i = 0; i < d->n_layers; ++i)
            QLX_REQUIRE(blobs[i] != nullptr, QLX_EINVAL, "blobs[" + std::to_string(i) + "] is NULL");
        const int fd = open(path, O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644);
        QLX_REQUIRE(fd >= 0, QLX_EIO, std::string("cannot create ") + path + ": " + errstr(errno));
        std::vector<char> pad(size_t(stride - blob_bytes), 0);
        auto put = [&](const char* p, uint64_t n) {
            while (n > 0) {
                const ssize_t r = write(fd, p, size_t(std::min<uint64_t>(n, 1ull << 30)));
                if (r < 0 && errno == EINTR) continue;
                if (r <= 0) {
                    const int e = errno;
                    close(fd);
                    throw Error{QLX_EIO, std::string("writing ") + path + ": " + errstr(e)};
                }
                p += r;
                n -= uint64_t(r);
            }
        };
        for (int i = 0; i < d->n_layers; ++i) {
            put(static_cast<const char*>(blobs[i]), blob_bytes);
            put(pad.data(), pad.size());
        }
        const int synced = fsync(fd);
        const int e = errno;
        close(fd);
        QLX_REQUIRE(synced == 0, QLX_EIO, std::string("fsync ") + path + ": " + errstr(e));
    });
}

int qlx_layer_file_open(qlx_layer_file** out, const char* path, const qlx_dims* d, int flags) {
    return guarded([&] {
        REQ_PTR(out, "out");
        REQ_PTR(path, "path");
        validate_dims(d);
        QLX_REQUIRE((flags & ~(QLX_FILE_BUFFERED | QLX_FILE_WIRE)) == 0, QLX_EINVAL, "unknown layer-file flags");
        *out = nullptr;
        const int form = (flags & QLX_FILE_WIRE) ? QLX_BLOB_WIRE : QLX_BLOB_FULL;
        uint64_t blob_bytes = 0;
        const uint64_t stride = stride_of(*d, form, &blob_bytes);
        int fd = -1;
        bool direct = false;
        if (!(flags & QLX_FILE_BUFFERED)) {
            fd = open(path, O_RDONLY | O_DIRECT | O_CLOEXEC);
            direct = fd >= 0;
        }
        if (fd < 0) fd = open(path, O_RDONLY | O_CLOEXEC);
        QLX_REQUIRE(fd >= 0, QLX_EIO, std::string("cannot open ") + path + ": " + errstr(errno));
        struct stat stt;
        if (fstat(fd, &stt) != 0 || uint64_t(stt.st_size) < stride * uint64_t(d->n_layers)) {
            const uint64_t have = fstat(fd, &stt) == 0 ? uint64_t(stt.st_size) : 0;
            close(fd);
            throw Error{QLX_EIO, std::string(path) + " holds " + std::to_string(have) + " bytes; " +
                                     std::to_string(d->n_layers) + " layers need " +
                                     std::to_string(stride * uint64_t(d->n_layers))};
        }
        if (direct) {
            // some file systems take O_DIRECT at open and refuse the reads
            void* probe = nullptr;
            QLX_REQUIRE(posix_memalign(&probe, kFileAlign, kFileAlign) == 0, QLX_EIO, "out of host memory");
            const ssize_t r = pread(fd, probe, kFileAlign, 0);
            std::free(probe);
            if (r != ssize_t(kFileAlign)) {
                close(fd);
                fd = open(path, O_RDONLY | O_CLOEXEC);
                QLX_REQUIRE(fd >= 0, QLX_EIO, std::string("cannot open ") + path + ": " + errstr(errno));
                direct = false;
            }
        }
        qlx_layer_file* f = new qlx_layer_file();
        f->path = path;
        f->fd = fd;
        f->direct = direct;
        f->dims = *d;
        f->form = form;
        f->blob_bytes = blob_bytes;
        f->stride = stride;
        // QLX_FILE_READERS (1..64) overrides the reader count (requests in flight)
        int readers = kReaders;
        if (const char* e = std::getenv("QLX_FILE_READERS")) readers = std::max(1, std::min(64, std::atoi(e)));
        for (int k = 0; k < readers; ++k) f->workers.emplace_back(reader, f);
        *out = f;
    });
}

int qlx_layer_file_close(qlx_layer_file* f) {
    return guarded([&] {
        if (!f) return;
        QLX_REQUIRE(f->attached == 0, QLX_EINVAL,
                    "layer file is still attached to " + std::to_string(f->attached) +
                        " context(s): detach it (qlx_ctx_set_layer_source(ctx, NULL)) first");
        close_file(f);
    });
}

int qlx_layer_file_info(const qlx_layer_file* f, int* direct, uint64_t* stride) {
    return guarded([&] {
        REQ_PTR(f, "file");
        if (direct) *direct = f->direct ? 1 : 0;
        if (stride) *stride = f->stride;
    });
}

int qlx_layer_file_read(qlx_layer_file* f, int layer, void* dst) {
    return guarded([&] {
        REQ_PTR(f, "file");
        REQ_PTR(dst, "dst");
        void* bounce = nullptr;
        QLX_REQUIRE(posix_memalign(&bounce, kFileAlign, size_t(f->stride)) == 0, QLX_EIO, "out of host memory");
        try {
            layer_file_read(f, layer, bounce);
        } catch (...) {
            std::free(bounce);
            throw;
        }
        std::memcpy(dst, bounce, size_t(f->blob_bytes));
        std::free(bounce);
    });
}

int qlx_stream_source_auto(uint64_t stack_bytes, uint64_t reserve_bytes, int* mode) {
    return guarded([&] {
        REQ_PTR(mode, "mode");
        uint64_t avail_kb = 0;
        FILE* fp = std::fopen("/proc/meminfo", "r");
        QLX_REQUIRE(fp != nullptr, QLX_EIO, "cannot read /proc/meminfo");
        char line[256];
        bool found = false;
        while (std::fgets(line, sizeof line, fp)) {
            unsigned long long kb = 0;
            if (std::sscanf(line, "MemAvailable: %llu kB", &kb) == 1) {
                avail_kb = kb;
                found = true;
                break;
            }
        }
        std::fclose(fp);
        QLX_REQUIRE(found, QLX_EIO, "/proc/meminfo has no MemAvailable line");
        const uint64_t avail = avail_kb * 1024;
        *mode = (stack_bytes <= avail && reserve_bytes <= avail - stack_bytes) ? QLX_STREAMED : QLX_STREAMED_DISK;
    });
}

}  // extern "C"
