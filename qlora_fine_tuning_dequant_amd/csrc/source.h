// Disk stream source: the stack file a layer stream reads when the frozen
// base does not stay in host RAM (internal; the C ABI is in qlx.h).
#pragma once
#include <condition_variable>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "qlx_internal.h"

namespace qlx {
constexpr int kStaging = 2;                 // pinned staging buffers per file
constexpr uint64_t kFileAlign = 4096;       // blob stride and direct-I/O alignment
constexpr uint64_t kReadChunk = 8ull << 20; // one pread job
constexpr int kReaders = 16;                // reader threads per file
}  // namespace qlx

struct qlx_layer_file {
    std::string path;
    int fd = -1;
    bool direct = false;  // O_DIRECT: reads bypass the page cache
    qlx_dims dims{};
    int form = 0;  // QLX_BLOB_FULL or QLX_BLOB_WIRE
    uint64_t blob_bytes = 0, stride = 0;

    // reader pool: a layer read is split into kReadChunk jobs
    struct Job {
        char* dst;
        uint64_t off, len;
    };
    std::vector<std::thread> workers;
    std::mutex mu;
    std::condition_variable cv_job, cv_done;
    std::deque<Job> jobs;
    int pending = 0;
    int io_errno = 0;
    bool short_read = false;
    bool stop = false;

    // pinned staging ring, bound to one device by qlx_ctx_set_layer_source
    int device = -1;
    int attached = 0;  // contexts that hold this file (qlx_ctx_set_layer_source)
    char* staging[qlx::kStaging] = {};
    hipEvent_t staging_free[qlx::kStaging] = {};
    int next = 0;
};

namespace qlx {
// Reads layer i's padded blob (f->stride bytes) into dst (kFileAlign-aligned,
// at least f->stride bytes) on the reader threads; returns when it is all
// there. Throws QLX_EIO on a failed or short read.
void layer_file_read(qlx_layer_file* f, int layer, void* dst);
}  // namespace qlx
