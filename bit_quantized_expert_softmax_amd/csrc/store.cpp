// Expert file store: blobs read from a file with parallel pread.
//
// "Show HN: mecanismo de código aberto executando Gemma 4 26B em 2 GB de RAM
// em qualquer Mac com série M", section "Abordagem técnica (MoE + streaming
// por SSD)": the experts a token needs are streamed from the SSD, and
// parallel pread (rather than mmap) brought one expert's read down to a few
// milliseconds. The file holds the blobs in the order [layer][expert], each
// padded to a whole number of 16 KiB pages (the padded size is the printed
// per-expert figure), so every blob starts on a page boundary and can be read
// unbuffered (O_DIRECT) in page-aligned parts.
//
// A store owns a fixed pool of reader threads. A read splits each requested
// blob into one page-aligned part per reader and returns when every part is
// in; reads of one store are serialised. Unbuffered reads need destination
// memory that the kernel can pin for the transfer; pinned memory of the GPU
// runtime is not (the read fails with EFAULT), so then each reader reads into
// its own aligned bounce buffer and copies out.
#include <errno.h>
#include <fcntl.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <thread>
#include <vector>

#include "host_common.h"
#include "moedecode.h"

using moe::fail;

namespace {
constexpr int64_t kPage = 16384;  // blob alignment in the file
constexpr int64_t kDirectAlign = 4096;
}  // namespace

struct moe_store {
  int fd = -1;
  int n_layers = 0, n_experts = 0;
  int64_t blob = 0, stride = 0;
  bool direct = false;
  std::atomic<bool> bounce{false};    // unbuffered reads go through bounce buffers
  std::vector<uint8_t*> bounce_buf;  // one per reader, part_max bytes, 4096-aligned
  size_t part_max = 0;
  std::vector<std::thread> readers;
  std::mutex call_mu;  // one read at a time
  std::mutex mu;
  std::condition_variable cv_work, cv_done;
  struct Part {
    int64_t off;
    size_t len;
    uint8_t* dst;
  };
  std::vector<Part> parts;
  size_t next = 0, done = 0;
  int err = 0;       // first errno of the current read
  bool short_read = false;
  bool stop = false;

  // pread of len bytes at off into dst; < 0: errno
  ssize_t read_part(int reader, uint8_t* dst, size_t len, int64_t off) {
    if (!bounce.load(std::memory_order_relaxed)) {
      const ssize_t r = pread(fd, dst, len, static_cast<off_t>(off));
      if (r >= 0 || errno != EFAULT || !direct) return r;
      bounce.store(true, std::memory_order_relaxed);
    }
    const ssize_t r = pread(fd, bounce_buf[reader], len, static_cast<off_t>(off));
    if (r > 0) memcpy(dst, bounce_buf[reader], static_cast<size_t>(r));
    return r;
  }

  void run(int reader) {
    for (;;) {
      Part p{};
      {
        std::unique_lock<std::mutex> lk(mu);
        cv_work.wait(lk, [&] { return stop || next < parts.size(); });
        if (stop) return;
        p = parts[next++];
      }
      int e = 0;
      bool sh = false;
      size_t got = 0;
      while (got < p.len) {
        const ssize_t r = read_part(reader, p.dst + got, p.len - got, p.off + static_cast<int64_t>(got));
        if (r < 0) {
          if (errno == EINTR) continue;
          e = errno;
          break;
        }
        if (r == 0) {
          sh = true;
          break;
        }
        got += static_cast<size_t>(r);
      }
      std::lock_guard<std::mutex> lk(mu);
      if (e && !err) err = e;
      if (sh) short_read = true;
      if (++done == parts.size()) cv_done.notify_all();
    }
  }
};

namespace moe {
bool store_fits(const moe_store* s, int layer, int n_experts, int64_t blob_bytes) {
  return s && layer >= 0 && layer < s->n_layers && s->n_experts == n_experts && s->blob == blob_bytes;
}
}  // namespace moe

extern "C" {

int64_t moe_store_stride(int64_t blob_bytes) {
  return blob_bytes <= 0 ? 0 : (blob_bytes + kPage - 1) / kPage * kPage;
}

moe_status moe_store_open(const char* path, int32_t n_layers, int32_t n_experts, int64_t blob_bytes,
                          int32_t threads, int32_t direct, moe_store** out) {
  moe::clear_error();
  const char* fn = "moe_store_open";
  if (!path || !out) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  *out = nullptr;
  if (n_layers < 1 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS || blob_bytes < 1)
    return fail(MOE_ESHAPE, "%s: n_layers %d, n_experts %d, blob_bytes %lld out of range", fn, n_layers,
                n_experts, static_cast<long long>(blob_bytes));
  if (threads < 1 || threads > 64) return fail(MOE_EINVAL, "%s: threads %d outside [1, 64]", fn, threads);
  const int64_t stride = moe_store_stride(blob_bytes);
  int fd = -1;
  bool is_direct = false;
  if (direct) {
    fd = open(path, O_RDONLY | O_DIRECT | O_CLOEXEC);
    is_direct = fd >= 0;
  }
  // file systems without unbuffered reads (tmpfs) refuse O_DIRECT: read buffered
  if (fd < 0) fd = open(path, O_RDONLY | O_CLOEXEC);
  if (fd < 0) return fail(MOE_EINVAL, "%s: cannot open %s: %s", fn, path, strerror(errno));
  struct stat st {};
  if (fstat(fd, &st) != 0 || st.st_size < static_cast<off_t>(stride) * n_layers * n_experts) {
    close(fd);
    return fail(MOE_ESHAPE, "%s: %s holds %lld bytes, %d x %d blobs of stride %lld need %lld", fn, path,
                static_cast<long long>(st.st_size), n_layers, n_experts, static_cast<long long>(stride),
                static_cast<long long>(stride) * n_layers * n_experts);
  }
  moe_store* s = new moe_store();
  s->fd = fd;
  s->n_layers = n_layers;
  s->n_experts = n_experts;
  s->blob = blob_bytes;
  s->stride = stride;
  s->direct = is_direct;
  if (is_direct) {
    const int64_t pages = stride / kPage;
    s->part_max = static_cast<size_t>((pages + threads - 1) / threads * kPage);
    for (int i = 0; i < threads; ++i) {
      void* b = nullptr;
      if (posix_memalign(&b, kDirectAlign, s->part_max) != 0) {
        for (uint8_t* q : s->bounce_buf) free(q);
        close(fd);
        delete s;
        return fail(MOE_ENOMEM, "%s: bounce buffers", fn);
      }
      s->bounce_buf.push_back(static_cast<uint8_t*>(b));
    }
  }
  for (int i = 0; i < threads; ++i) s->readers.emplace_back([s, i] { s->run(i); });
  *out = s;
  return MOE_OK;
}

int32_t moe_store_is_direct(const moe_store* s) { return s && s->direct ? 1 : 0; }

void moe_store_close(moe_store* s) {
  if (!s) return;
  {
    std::lock_guard<std::mutex> lk(s->mu);
    s->stop = true;
  }
  s->cv_work.notify_all();
  for (auto& t : s->readers) t.join();
  for (uint8_t* b : s->bounce_buf) free(b);
  if (s->fd >= 0) close(s->fd);
  delete s;
}

moe_status moe_store_read(moe_store* s, int32_t layer, const int32_t* experts, int32_t n, void* const* dst) {
  moe::clear_error();
  const char* fn = "moe_store_read";
  if (!s) return fail(MOE_EINVAL, "%s: NULL handle", fn);
  if (n < 0 || n > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "%s: n = %d", fn, n);
  if (n == 0) return MOE_OK;
  if (!experts || !dst) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  if (layer < 0 || layer >= s->n_layers) return fail(MOE_EINVAL, "%s: layer %d outside [0, %d)", fn, layer, s->n_layers);
  for (int i = 0; i < n; ++i) {
    if (experts[i] < 0 || experts[i] >= s->n_experts)
      return fail(MOE_EINVAL, "%s: expert %d outside [0, %d)", fn, experts[i], s->n_experts);
    if (!dst[i]) return fail(MOE_EINVAL, "%s: dst[%d] is NULL", fn, i);
    if (s->direct && reinterpret_cast<uintptr_t>(dst[i]) % kDirectAlign)
      return fail(MOE_EALIGN, "%s: dst[%d] must be %lld-byte aligned for unbuffered reads", fn, i,
                  static_cast<long long>(kDirectAlign));
  }
  std::lock_guard<std::mutex> call(s->call_mu);
  // one page-aligned part per reader and blob (the padded stride is read
  // whole, so unbuffered reads see aligned offsets and lengths)
  const int64_t pages = s->stride / kPage;
  const int64_t nr = static_cast<int64_t>(s->readers.size());
  const int64_t per = (pages + nr - 1) / nr;
  std::vector<moe_store::Part> parts;
  for (int i = 0; i < n; ++i) {
    const int64_t base = (static_cast<int64_t>(layer) * s->n_experts + experts[i]) * s->stride;
    for (int64_t p0 = 0; p0 < pages; p0 += per) {
      const int64_t np = p0 + per < pages ? per : pages - p0;
      parts.push_back({base + p0 * kPage, static_cast<size_t>(np * kPage), static_cast<uint8_t*>(dst[i]) + p0 * kPage});
    }
  }
  int err;
  bool sh;
  {
    std::unique_lock<std::mutex> lk(s->mu);
    s->parts.swap(parts);
    s->next = s->done = 0;
    s->err = 0;
    s->short_read = false;
    s->cv_work.notify_all();
    s->cv_done.wait(lk, [&] { return s->done == s->parts.size(); });
    err = s->err;
    sh = s->short_read;
    s->parts.clear();
    s->next = s->done = 0;
  }
  if (err) return fail(MOE_EINVAL, "%s: pread failed: %s", fn, strerror(err));
  if (sh) return fail(MOE_ESHAPE, "%s: the file ended inside a blob", fn);
  return MOE_OK;
}

}  // extern "C"
