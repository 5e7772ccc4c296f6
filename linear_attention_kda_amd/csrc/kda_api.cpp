// C ABI of the KDA forward pass: host-side validation, launch planning, errors.
// The argument rules follow the kernel API the pages describe
// [trend.ondo.sh "MoonshotAI/FlashKDA", section "커널 API와 제약 조건"]:
// K = V = 128, cu_seqlens only with B = 1, states bf16/fp32/absent with
// matching dtypes.  Rejection reasons are kept as text per thread and, with
// KDA_LOG=1 in the environment, printed to stderr.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>
#include <thread>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("KDA_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

kda_status fail(kda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (log_enabled()) std::fprintf(stderr, "[kda] rejected: %s (%s)\n", buf, kda_status_string(st));
  return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kda_status validate(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    const void* s0, int s0_dtype, const void* s1, int s1_dtype, const int32_t* cu,
                    int32_t num_seqs, int32_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                    const void* out, int32_t* n_out, bool g_scalar) {
  if (K != V || (K != 64 && K != KDA_HEAD_DIM && K != 256))
    return fail(KDA_ERR_HEAD_DIM, "K=%d V=%d: K = V in {64, 128, 256} is required", K, V);
  if (B <= 0 || H <= 0 || T < 0)
    return fail(KDA_ERR_SHAPE, "invalid sizes B=%d T=%lld H=%d", B, (long long)T, H);
  if (cu != nullptr) {
    if (B != 1) return fail(KDA_ERR_VARLEN_BATCH, "cu_seqlens requires B = 1 (got B=%d)", B);
    if (num_seqs <= 0) return fail(KDA_ERR_SHAPE, "cu_seqlens given with num_seqs=%d", num_seqs);
  }
  const int32_t N = cu ? num_seqs : B;
  if (s0 != nullptr && s0_dtype != KDA_BF16 && s0_dtype != KDA_FP32)
    return fail(KDA_ERR_DTYPE, "initial_dtype=%d is not KDA_BF16 or KDA_FP32", s0_dtype);
  if (s1 != nullptr && s1_dtype != KDA_BF16 && s1_dtype != KDA_FP32)
    return fail(KDA_ERR_DTYPE, "final_dtype=%d is not KDA_BF16 or KDA_FP32", s1_dtype);
  if (s0 != nullptr && s1 != nullptr && s0_dtype != s1_dtype)
    return fail(KDA_ERR_STATE_DTYPE, "initial_state dtype %d differs from final_state dtype %d",
                s0_dtype, s1_dtype);
  // sizes: element counts must fit int64, workgroup counts int32
  const long double elems = (long double)B * (long double)T * (long double)H * K;
  if (elems > (long double)(INT64_MAX / 4))
    return fail(KDA_ERR_SHAPE, "tensor size overflows 64-bit indexing");
  if ((int64_t)N * H * 2 > (int64_t)INT_MAX - 64)
    return fail(KDA_ERR_SHAPE, "N*H=%lld too large", (long long)N * H);
  // a chunk's rows of every head stay within 32-bit buffer offsets
  if ((int64_t)H * K > (int64_t)1 << 22)
    return fail(KDA_ERR_SHAPE, "H*K=%lld too large (at most 4194304)", (long long)H * K);
  if (T > 0) {
    if (!q || !k || !v || !g || !beta || !out)
      return fail(KDA_ERR_NULL, "q, k, v, g, beta and out are required when T > 0");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
      return fail(KDA_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
    if (!aligned(g, g_scalar ? 4 : 16))
      return fail(KDA_ERR_ALIGN, "g must be %d-byte aligned", g_scalar ? 4 : 16);
    if (!aligned(beta, 4)) return fail(KDA_ERR_ALIGN, "beta must be 4-byte aligned");
  }
  if ((s0 && !aligned(s0, 16)) || (s1 && !aligned(s1, 16)))
    return fail(KDA_ERR_ALIGN, "states must be 16-byte aligned");
  if (n_out) *n_out = N;
  return KDA_OK;
}

int device_cu_count(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return 0;
}

int forced_splits() {
  const char* e = std::getenv("KDA_VSPLIT");
  if (e != nullptr && (e[0] == '1' || e[0] == '2') && e[1] == '\0') return e[0] - '0';
  return 0;
}

int seg_min_chunks() {
  const char* e = std::getenv("KDA_SEG_MIN");
  if (e != nullptr && e[0] != '\0') {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v <= (1L << 30)) return (int)v;
  }
  return kda::kSegMinDefault;
}

bool seq_split_enabled() {
  const char* e = std::getenv("KDA_SEQSPLIT");
  return !(e != nullptr && e[0] == '0' && e[1] == '\0');
}

// The device's segment length for N equal sequences of c chunks (fixed-length
// batches) with emax state slots and ucap fix-up units, or 0 when it does not
// split them.  Same rule as the kernels' plan.
int64_t fixed_length_segment(int64_t N, int64_t c, int64_t H, int64_t cus, int seg_min,
                             int64_t emax, int64_t ucap) {
  if (c <= seg_min || emax <= 0) return 0;
  auto fits = [&](int64_t m) {
    const int64_t extra = c > m ? N * (c - m) : 0;
    const int64_t slots = c > m ? N * ((c - 1) / m) : 0;
    return kda::kSlackDen * H * (N * c + extra) <= kda::kSlackNum * m * cus && slots <= emax &&
           H * extra <= ucap;
  };
  if (!fits(c)) return 0;
  int64_t lo = seg_min, hi = c;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (fits(mid)) hi = mid;
    else lo = mid + 1;
  }
  return hi < c ? hi : 0;
}

struct LaunchPlan {
  int nsplit;     // value-column slices per (sequence, head)
  int emax;       // segment state slots (0: no sequence splitting)
  int ucap;       // fix-up units (one 64 x 128 output block each)
  int seg_min;
  int64_t workgroups;
  size_t workspace;
};

// rows: packed rows (T with cu_seqlens, else B*T); T: tokens per row, or the
// packed total with cu_seqlens.  cap_bytes > 0 bounds the workspace (a
// caller-provided buffer): the state slots and fix-up units are then sized to
// it, and the device plan splits sequences only as far as they fit.
LaunchPlan make_plan(int32_t N, int64_t T, int32_t H, bool varlen, int32_t cus,
                     size_t cap_bytes = 0, bool value_split = true) {
  LaunchPlan lp{};
  lp.seg_min = seg_min_chunks();
  const int forced = value_split ? forced_splits() : 0;
  const int64_t c_max = (T + KDA_CHUNK - 1) / KDA_CHUNK;  // chunks of the longest possible sequence
  int64_t emax = 0, ucap = 0;
  // the device plan counts chunks and fix-up units in 32-bit integers
  const int64_t chunks = (varlen ? c_max + N : (int64_t)N * c_max);
  const bool small_enough = chunks < (1LL << 30) && chunks * H < (1LL << 30);
  if (seq_split_enabled() && forced != 2 && N <= kda::kSortLimit && c_max > lp.seg_min &&
      small_enough) {
    emax = std::min(kda::workspace_slots(cus, H), 512);
    ucap = chunks * H;  // every chunk past a first segment, at most
    if (cap_bytes > 0) {  // slots first (at most half the buffer), then fix-up blocks
      const size_t slot = kda::workspace_slot_bytes(H);
      emax = std::min<int64_t>(emax, (int64_t)(cap_bytes / 2 / slot));
      const size_t rest = cap_bytes - kda::workspace_layout(0, H, (int)emax).total;
      ucap = std::min<int64_t>(ucap, (int64_t)(rest / kda::kUnitBytes) - 1);
      if (ucap < H) emax = 0;  // not one chunk of every head fits
    }
    if (emax > 0 && !varlen) {  // the host knows the device's plan exactly: size to it
      const int64_t M = fixed_length_segment(N, c_max, H, cus, lp.seg_min, emax, ucap);
      if (M == 0) {
        emax = 0;
      } else {
        emax = N * ((c_max - 1) / M);
        ucap = H * N * (c_max - M);
      }
    }
  }
  if (emax <= 0) emax = ucap = 0;
  lp.emax = (int)emax;
  lp.ucap = (int)ucap;
  // one workgroup per (sequence, head) already covers the CUs: no value split
  lp.nsplit = forced ? forced : (!value_split || emax > 0 || (int64_t)N * H >= cus) ? 1 : 2;
  if (emax > 0 && lp.nsplit != 1) lp.emax = lp.ucap = 0;
  const int64_t groups = (int64_t)N + (lp.emax > 0 ? 2 * (int64_t)lp.emax : 0);
  lp.workgroups = (groups * H + 7) / 8 * 8 * lp.nsplit;
  lp.workspace = lp.emax > 0 ? kda::workspace_layout(lp.ucap, H, lp.emax).total : 0;
  return lp;
}

// Library-owned stream-ordered pool, one per device, for the workspaces too large
// to keep between calls (see Workspace below).  It keeps up to kPoolKeepBytes
// reserved (so a repeated call of the same size maps no new device memory) and
// hands anything above that back at the next synchronisation.
constexpr uint64_t kPoolKeepBytes = 2ull << 30;

hipError_t workspace_pool(hipMemPool_t* out) {
  static std::mutex mu;
  static hipMemPool_t pools[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (pools[dev] == nullptr) {
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof props);
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    err = hipMemPoolCreate(&pool, &props);
    if (err != hipSuccess) return err;
    uint64_t keep = kPoolKeepBytes;
    err = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (err != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return err;
    }
    pools[dev] = pool;
  }
  *out = pools[dev];
  return hipSuccess;
}

// A second stream per device, created on first use (default priority), on which
// the backward's checkpointing forward pass runs beside the chunk-local tiles.
hipError_t side_stream(hipStream_t* out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (streams[dev] == nullptr) {
    err = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking);
    if (err != hipSuccess) {
      streams[dev] = nullptr;
      return err;
    }
  }
  *out = streams[dev];
  return hipSuccess;
}

// Workspaces kept between calls.  Taken from the pool per call, a workspace made
// the next call's hipMallocFromPoolAsync wait on the host until the previous
// call's kernels had finished; an event recorded per call to order reuse across
// streams costs the device a few microseconds between calls.  A workspace is
// therefore kept per stream and reused by later calls on that stream, which the
// stream itself orders: a call enqueues no synchronisation of its own.  The
// per-thread default stream is one handle for many streams, so its buffers are
// also keyed by the calling thread.  At most kCacheEntries buffers of
// kCacheBytes in total are kept per device.  A buffer that must grow is freed
// after its stream has drained (host wait); when a new stream's buffer does not
// fit, every kept buffer is freed after the device has drained.  Larger
// workspaces come from the pool for the one call.  A lease holds its device's
// lock from acquire() to release(), i.e. while the call enqueues its work.
constexpr size_t kCacheBytes = 2ull << 30;
constexpr size_t kCacheGrain = 32ull << 20;
constexpr int kCacheEntries = 4;

struct CacheEntry {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipStream_t stream = nullptr;
  std::thread::id thread;  // set for the per-thread default stream only
};

struct DeviceCache {
  std::mutex mu;
  CacheEntry e[kCacheEntries];
};

DeviceCache g_cache[64];

// Frees every kept buffer of a device once the device has drained.
hipError_t drop_all(DeviceCache& c) {
  bool any = false;
  for (const CacheEntry& x : c.e) any = any || x.ptr != nullptr;
  if (!any) return hipSuccess;
  hipError_t err = hipDeviceSynchronize();
  for (CacheEntry& x : c.e) {
    if (x.ptr != nullptr) {
      const hipError_t e = hipFree(x.ptr);
      if (err == hipSuccess) err = e;
    }
    x = CacheEntry{};
  }
  return err;
}

class Workspace {
 public:
  Workspace() = default;
  Workspace(const Workspace&) = delete;
  Workspace& operator=(const Workspace&) = delete;
  ~Workspace() { (void)release(); }

  // A workspace of at least `bytes` bytes for work enqueued on `hs`.
  hipError_t acquire(size_t bytes, hipStream_t hs) {
    hs_ = hs;
    if (bytes == 0) return hipSuccess;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    const size_t need = (bytes + kCacheGrain - 1) / kCacheGrain * kCacheGrain;
    if (need <= kCacheBytes) {
      DeviceCache& c = g_cache[dev];
      lock_ = std::unique_lock<std::mutex>(c.mu);
      const std::thread::id tid =
          hs == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
      CacheEntry* mine = nullptr;
      size_t total = 0;
      for (CacheEntry& x : c.e) {
        total += x.bytes;
        if (x.ptr != nullptr && x.stream == hs && x.thread == tid) mine = &x;
      }
      if (mine != nullptr && mine->bytes < need) {  // grow: free after this stream's work
        err = hipStreamSynchronize(hs);
        const hipError_t e = hipFree(mine->ptr);
        if (err == hipSuccess) err = e;
        total -= mine->bytes;
        *mine = CacheEntry{};
        if (err != hipSuccess) {
          lock_.unlock();
          return err;
        }
        mine = nullptr;
      }
      if (mine == nullptr) {
        CacheEntry* slot = nullptr;
        for (CacheEntry& x : c.e)
          if (x.ptr == nullptr) { slot = &x; break; }
        if (slot == nullptr || total + need > kCacheBytes) {
          err = drop_all(c);
          slot = &c.e[0];
          if (err != hipSuccess) {
            lock_.unlock();
            return err;
          }
        }
        err = hipMalloc(&slot->ptr, need);
        if (err != hipSuccess) {
          *slot = CacheEntry{};
          lock_.unlock();
          return err;
        }
        slot->bytes = need;
        slot->stream = hs;
        slot->thread = tid;
        mine = slot;
      }
      ptr_ = mine->ptr;
      return hipSuccess;
    }
    hipMemPool_t pool = nullptr;
    err = workspace_pool(&pool);
    if (err == hipSuccess) err = hipMallocFromPoolAsync(&pooled_, bytes, pool, hs);
    if (err == hipErrorOutOfMemory) {
      // earlier calls' workspaces, freed on their streams, may still be held by the
      // pool until a synchronisation: wait for the device, hand them back, retry once
      (void)hipGetLastError();
      err = hipDeviceSynchronize();
      if (err == hipSuccess) err = hipMemPoolTrimTo(pool, 0);
      if (err == hipSuccess) err = hipMallocFromPoolAsync(&pooled_, bytes, pool, hs);
    }
    if (err != hipSuccess) pooled_ = nullptr;
    ptr_ = pooled_;
    return err;
  }

  void* ptr() const { return ptr_; }

  // Called once every launch of the call has been enqueued on the stream.
  hipError_t release() {
    hipError_t err = hipSuccess;
    if (pooled_ != nullptr) {
      err = hipFreeAsync(pooled_, hs_);
      pooled_ = nullptr;
    }
    ptr_ = nullptr;
    if (lock_.owns_lock()) lock_.unlock();
    return err;
  }

 private:
  std::unique_lock<std::mutex> lock_;
  void* ptr_ = nullptr;
  void* pooled_ = nullptr;
  hipStream_t hs_ = nullptr;
};

// Head dimension 256: per-chunk records in a workspace (kept between calls), then the
// serial state pass (no sequence splitting).
kda_status fwd_dim_impl(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, float scale, const void* initial_state,
                        int initial_dtype, void* final_state, int final_dtype,
                        const int32_t* cu_seqlens, int32_t N, int32_t B, int64_t T, int32_t H,
                        int32_t D, void* out, void* stream, bool g_scalar,
                        const kda::ExtWorkspace* ext) {
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t rows = cu_seqlens ? T : (int64_t)B * T;
  kda::DimParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = g;
  p.g_scalar = g_scalar ? 1 : 0;
  p.beta = beta;
  p.out = static_cast<uint16_t*>(out);
  p.s0 = initial_state;
  p.s1 = final_state;
  p.s0_fp32 = initial_dtype == KDA_FP32;
  p.s1_fp32 = final_dtype == KDA_FP32;
  p.cu = cu_seqlens;
  p.T = T;
  p.scale = scale;
  p.nseq = N;
  p.H = H;
  p.D = D;
  p.slots = rows > 0 ? kda::dim_slots(N, rows) : 0;
  const size_t bytes = (size_t)p.slots * H * kda::dim_record_bytes(D);
  Workspace ws;
  if (bytes > 0 && ext != nullptr) {
    if (bytes > ext->bytes)
      return fail(KDA_ERR_WORKSPACE,
                  "head dimension %d needs %zu bytes of per-chunk records, more than the %zu "
                  "bytes of the static scratch", D, bytes, ext->bytes);
    p.ws = static_cast<char*>(ext->ptr);
  } else if (bytes > 0) {
    const hipError_t e = ws.acquire(bytes, hs);
    if (e != hipSuccess)
      return fail(KDA_ERR_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    p.ws = static_cast<char*>(ws.ptr());
  }
  if (log_enabled())
    std::fprintf(stderr, "[kda] launch: %s D=%d N=%d H=%d T=%lld record_slots=%lld workspace=%zu%s\n",
                 g_scalar ? "gdn" : "kda", D, N, H, (long long)T, (long long)p.slots, bytes,
                 ext ? " (static scratch)" : "");
  const hipError_t err = kda::launch_fwd_dim(p, hs);
  const hipError_t e = ws.release();
  if (err == hipSuccess && e != hipSuccess)
    return fail(KDA_ERR_HIP, "workspace release: %s", hipGetErrorString(e));
  if (err != hipSuccess)
    return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return KDA_OK;
}

}  // namespace

namespace kda {

kda_status fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    float scale, const void* initial_state, int initial_dtype, void* final_state,
                    int final_dtype, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                    int64_t T, int32_t H, int32_t K, int32_t V, void* out, void* stream,
                    bool g_scalar, const ExtWorkspace* ext) {
  g_last_error.clear();
  int32_t N = 0;
  kda_status st = validate(q, k, v, g, beta, initial_state, initial_dtype, final_state,
                           final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out, &N,
                           g_scalar);
  if (st != KDA_OK) return st;
  if (T == 0 && final_state == nullptr) return KDA_OK;  // nothing observable to compute
  if (K == 256)
    return fwd_dim_impl(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state,
                        final_dtype, cu_seqlens, N, B, T, H, K, out, stream, g_scalar, ext);

  int cus = 0;
  if (device_cu_count(&cus) != 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count of the current device");
  // K = 64 runs the fused kernel in one 64-column slice per (sequence, head, segment)
  const LaunchPlan lp = make_plan(N, T, H, cu_seqlens != nullptr, cus, ext ? ext->bytes : 0,
                                  K == KDA_HEAD_DIM);
  const hipStream_t hs = static_cast<hipStream_t>(stream);

  kda::Params p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = g;
  p.g_scalar = g_scalar ? 1 : 0;
  p.beta = beta;
  p.out = static_cast<uint16_t*>(out);
  p.s0 = initial_state;
  p.s1 = final_state;
  p.s0_fp32 = initial_dtype == KDA_FP32;
  p.s1_fp32 = final_dtype == KDA_FP32;
  p.cu = cu_seqlens;
  p.T = T;
  p.scale = scale;
  p.nseq = N;
  p.H = H;
  p.dk = K;
  p.cus = cus;
  p.seg_min = lp.seg_min;
  Workspace ws;
  if (lp.emax > 0) {
    char* base = nullptr;
    if (ext != nullptr) {
      if (lp.workspace > ext->bytes)  // the plan is sized to the scratch: never taken
        return fail(KDA_ERR_WORKSPACE, "split plan needs %zu bytes, the static scratch holds %zu",
                    lp.workspace, ext->bytes);
      base = static_cast<char*>(ext->ptr);
    } else {
      const hipError_t e = ws.acquire(lp.workspace, hs);
      if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "workspace of %zu bytes: %s", lp.workspace, hipGetErrorString(e));
      base = static_cast<char*>(ws.ptr());
    }
    const kda::WorkspaceLayout wl = kda::workspace_layout(lp.ucap, H, lp.emax);
    p.emax = lp.emax;
    p.ucap = lp.ucap;
    p.o0 = reinterpret_cast<uint16_t*>(base + wl.o0);
    p.st = reinterpret_cast<float*>(base + wl.st);
    p.sb = reinterpret_cast<uint16_t*>(base + wl.sb);
    p.state_flags = reinterpret_cast<int*>(base + wl.flag);
  }
  if (log_enabled())
    std::fprintf(stderr,
                 "[kda] launch: %s D=%d N=%d H=%d T=%lld value_splits=%d cus=%d varlen=%d "
                 "segment_slots=%d fixup_units=%d workspace=%zu%s\n",
                 g_scalar ? "gdn" : "kda", K, N, H, (long long)T, lp.nsplit, cus,
                 cu_seqlens != nullptr, lp.emax, lp.ucap, lp.workspace,
                 ext ? " (static scratch)" : "");
  const hipError_t err = kda::launch_fwd(p, lp.nsplit, hs);
  const hipError_t e = ws.release();
  if (err == hipSuccess && e != hipSuccess)
    return fail(KDA_ERR_HIP, "workspace release: %s", hipGetErrorString(e));
  if (err != hipSuccess)
    return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return KDA_OK;
}

kda_status record_failure(kda_status st, const char* text) { return fail(st, "%s", text); }

}  // namespace kda

extern "C" {

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "required pointer is NULL";
    case KDA_ERR_HEAD_DIM: return "unsupported head dimension";
    case KDA_ERR_VARLEN_BATCH: return "cu_seqlens requires B = 1";
    case KDA_ERR_STATE_DTYPE: return "initial and final state dtypes differ";
    case KDA_ERR_DTYPE: return "invalid dtype";
    case KDA_ERR_SHAPE: return "invalid sizes";
    case KDA_ERR_ALIGN: return "misaligned pointer";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_WORKSPACE: return "call needs more workspace than the static scratch holds";
    default: return "unknown status";
  }
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

kda_status kda_release_workspaces(void) {
  g_last_error.clear();
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess && (dev < 0 || dev >= 64)) err = hipErrorInvalidDevice;
  if (err == hipSuccess) {
    DeviceCache& c = g_cache[dev];
    std::lock_guard<std::mutex> lock(c.mu);
    err = drop_all(c);
  }
  if (err != hipSuccess)
    return fail(KDA_ERR_HIP, "releasing the workspaces: %s", hipGetErrorString(err));
  return KDA_OK;
}

kda_status kda_fwd_check(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, const void* initial_state,
                         int initial_dtype, const void* final_state, int final_dtype,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                         int32_t H, int32_t K, int32_t V, const void* out) {
  (void)scale;
  g_last_error.clear();
  return validate(q, k, v, g, beta, initial_state, initial_dtype, final_state, final_dtype,
                  cu_seqlens, num_seqs, B, T, H, K, V, out, nullptr, false);
}

kda_status kda_gdn_fwd_check(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, float scale, const void* initial_state,
                             int initial_dtype, const void* final_state, int final_dtype,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                             int32_t H, int32_t K, int32_t V, const void* out) {
  (void)scale;
  g_last_error.clear();
  return validate(q, k, v, g, beta, initial_state, initial_dtype, final_state, final_dtype,
                  cu_seqlens, num_seqs, B, T, H, K, V, out, nullptr, true);
}

kda_status kda_plan(int32_t n_sequences, int64_t T, int32_t H, int32_t varlen, int32_t cu_count,
                    int32_t* workgroups, int32_t* value_splits, int64_t* workspace_bytes) {
  g_last_error.clear();
  if (!workgroups || !value_splits || !workspace_bytes)
    return fail(KDA_ERR_NULL, "kda_plan outputs are NULL");
  if (n_sequences <= 0 || H <= 0 || T < 0)
    return fail(KDA_ERR_SHAPE, "kda_plan: N=%d T=%lld H=%d", n_sequences, (long long)T, H);
  int cus = cu_count;
  if (cus <= 0 && device_cu_count(&cus) != 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count of the current device");
  const LaunchPlan lp = make_plan(n_sequences, T, H, varlen != 0, cus);
  *value_splits = lp.nsplit;
  *workgroups = (int32_t)lp.workgroups;
  *workspace_bytes = (int64_t)lp.workspace;
  return KDA_OK;
}

kda_status kda_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   float scale, const void* initial_state, int initial_dtype, void* final_state,
                   int final_dtype, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                   int64_t T, int32_t H, int32_t K, int32_t V, void* out, void* stream) {
  return kda::fwd_impl(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state,
                       final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out, stream, false,
                       nullptr);
}

kda_status kda_gdn_fwd(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float scale, const void* initial_state,
                       int initial_dtype, void* final_state, int final_dtype,
                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                       int32_t H, int32_t K, int32_t V, void* out, void* stream) {
  return kda::fwd_impl(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state,
                       final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out, stream, true,
                       nullptr);
}

}  // extern "C"

namespace {

kda_status validate_decode(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const void* state, int state_dtype,
                           const int32_t* state_indices, int32_t N, int32_t H, int32_t K,
                           int32_t V, const void* out, bool g_scalar) {
  if (K != V || (K != 64 && K != KDA_HEAD_DIM && K != 256))
    return fail(KDA_ERR_HEAD_DIM, "K=%d V=%d: K = V in {64, 128, 256} is required", K, V);
  if (N < 0 || H <= 0) return fail(KDA_ERR_SHAPE, "invalid sizes N=%d H=%d", N, H);
  if ((int64_t)N * H > (int64_t)INT_MAX)
    return fail(KDA_ERR_SHAPE, "N*H=%lld too large", (long long)N * H);
  if (state_dtype != KDA_BF16 && state_dtype != KDA_FP32)
    return fail(KDA_ERR_DTYPE, "state_dtype=%d is not KDA_BF16 or KDA_FP32", state_dtype);
  if (N > 0) {
    if (!q || !k || !v || !g || !beta || !out || !state)
      return fail(KDA_ERR_NULL, "q, k, v, g, beta, state and out are required when N > 0");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(state, 16))
      return fail(KDA_ERR_ALIGN, "q, k, v, out and state must be 16-byte aligned");
    if (!aligned(g, g_scalar ? 4 : 16))
      return fail(KDA_ERR_ALIGN, "g must be %d-byte aligned", g_scalar ? 4 : 16);
    if (!aligned(beta, 4) || (state_indices && !aligned(state_indices, 4)))
      return fail(KDA_ERR_ALIGN, "beta and state_indices must be 4-byte aligned");
  }
  return KDA_OK;
}

kda_status decode_impl(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float scale, void* state, int state_dtype,
                       const int32_t* state_indices, int32_t N, int32_t H, int32_t K, int32_t V,
                       void* out, void* stream, bool g_scalar) {
  g_last_error.clear();
  kda_status st = validate_decode(q, k, v, g, beta, state, state_dtype, state_indices, N, H, K,
                                  V, out, g_scalar);
  if (st != KDA_OK) return st;
  if (N == 0) return KDA_OK;
  kda::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = g;
  p.g_scalar = g_scalar ? 1 : 0;
  p.beta = beta;
  p.out = static_cast<uint16_t*>(out);
  p.state = state;
  p.idx = state_indices;
  p.scale = scale;
  p.state_fp32 = state_dtype == KDA_FP32;
  p.nseq = N;
  p.H = H;
  p.D = K;
  if (log_enabled())
    std::fprintf(stderr, "[kda] decode: %s N=%d H=%d state=%s indexed=%d\n", g_scalar ? "gdn" : "kda",
                 N, H, p.state_fp32 ? "fp32" : "bf16", state_indices != nullptr);
  const hipError_t err = kda::launch_decode(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(KDA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(err));
  return KDA_OK;
}


}  // namespace

extern "C" {

kda_status kda_decode_check(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, float scale, const void* state, int state_dtype,
                            const int32_t* state_indices, int32_t N, int32_t H, int32_t K,
                            int32_t V, const void* out) {
  (void)scale;
  g_last_error.clear();
  return validate_decode(q, k, v, g, beta, state, state_dtype, state_indices, N, H, K, V, out,
                         false);
}

kda_status kda_gdn_decode_check(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, float scale, const void* state, int state_dtype,
                                const int32_t* state_indices, int32_t N, int32_t H, int32_t K,
                                int32_t V, const void* out) {
  (void)scale;
  g_last_error.clear();
  return validate_decode(q, k, v, g, beta, state, state_dtype, state_indices, N, H, K, V, out,
                         true);
}

kda_status kda_decode(const void* q, const void* k, const void* v, const float* g,
                      const float* beta, float scale, void* state, int state_dtype,
                      const int32_t* state_indices, int32_t N, int32_t H, int32_t K, int32_t V,
                      void* out, void* stream) {
  return decode_impl(q, k, v, g, beta, scale, state, state_dtype, state_indices, N, H, K, V, out,
                     stream, false);
}

kda_status kda_gdn_decode(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, float scale, void* state, int state_dtype,
                          const int32_t* state_indices, int32_t N, int32_t H, int32_t K, int32_t V,
                          void* out, void* stream) {
  return decode_impl(q, k, v, g, beta, scale, state, state_dtype, state_indices, N, H, K, V, out,
                     stream, true);
}

}  // extern "C"

namespace {

kda_status validate_bwd(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const void* s0, int s0_dtype, const void* d_out,
                        const void* dsT, int dsT_dtype, const int32_t* cu, int32_t num_seqs,
                        int32_t B, int64_t T, int32_t H, int32_t K, int32_t V, const float* dq,
                        const float* dk, const float* dv, const float* dg, const float* dbeta,
                        const float* ds0, int32_t* n_out) {
  if (K != KDA_HEAD_DIM || V != KDA_HEAD_DIM)
    return fail(KDA_ERR_HEAD_DIM, "K=%d V=%d: the backward pass takes K = V = 128 only", K, V);
  kda_status st = validate(q, k, v, g, beta, s0, s0_dtype, nullptr, KDA_FP32, cu, num_seqs, B, T,
                           H, K, V, T > 0 ? d_out : nullptr, n_out, false);
  if (st != KDA_OK) return st;
  if (dsT != nullptr && dsT_dtype != KDA_BF16 && dsT_dtype != KDA_FP32)
    return fail(KDA_ERR_DTYPE, "d_final_dtype=%d is not KDA_BF16 or KDA_FP32", dsT_dtype);
  if (T > 0 && (!d_out || !dq || !dk || !dv || !dg || !dbeta))
    return fail(KDA_ERR_NULL, "d_out, dq, dk, dv, dg and dbeta are required when T > 0");
  if ((d_out && !aligned(d_out, 16)) || (dq && !aligned(dq, 16)) || (dk && !aligned(dk, 16)) ||
      (dv && !aligned(dv, 16)) || (dg && !aligned(dg, 16)) || (dsT && !aligned(dsT, 16)) ||
      (ds0 && !aligned(ds0, 16)))
    return fail(KDA_ERR_ALIGN, "d_out, gradients and states must be 16-byte aligned");
  if (dbeta && !aligned(dbeta, 4)) return fail(KDA_ERR_ALIGN, "dbeta must be 4-byte aligned");
  return KDA_OK;
}

// Chunk slots of the backward: sequence n's chunk c is slot n + floor(bos_n / 64) + c.
int64_t bwd_slots(int32_t N, int64_t rows) { return (int64_t)N + (rows + 63) / 64 + 1; }

// The backward's per-chunk tiles cover at most this many bytes at once; longer inputs
// go through in groups of chunk slots (KDA_BWD_GROUP_SLOTS sets the group size).
constexpr size_t kBwdGroupBytes = size_t(8) << 30;

int64_t bwd_group_slots(int32_t N, int64_t rows, int32_t H) {
  const int64_t slots = bwd_slots(N, rows);
  int64_t g = 0;
  const char* e = std::getenv("KDA_BWD_GROUP_SLOTS");
  if (e != nullptr && e[0] != '\0') g = std::strtoll(e, nullptr, 10);
  if (g < 1) g = (int64_t)(kBwdGroupBytes / ((size_t)H * kda::BwdTiles::floats_per_batch() * 4));
  return g < 1 ? 1 : g > slots ? slots : g;
}

// Workspace regions: one group's tiles, the checkpoints of every slot, two carry
// buffers when there is more than one group, the forward pass's outputs.
struct BwdLayout {
  size_t tiles, ckpt, carry, out, total;
};

BwdLayout bwd_layout(int32_t N, int64_t rows, int32_t H) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t slots = bwd_slots(N, rows), gs = bwd_group_slots(N, rows, H);
  BwdLayout l{};
  l.tiles = up((size_t)gs * H * kda::BwdTiles::floats_per_batch() * 4);
  l.ckpt = up((size_t)slots * H * kda::BwdTiles::ckpt_floats_per_batch() * 4);
  l.carry = gs < slots ? up((size_t)2 * H * 128 * 128 * 4) : 0;
  l.out = up((size_t)rows * H * 128 * 2);
  l.total = l.tiles + l.ckpt + l.carry + l.out;
  return l;
}

size_t bwd_workspace_bytes(int32_t N, int64_t rows, int32_t H) { return bwd_layout(N, rows, H).total; }

}  // namespace

extern "C" {

kda_status kda_bwd_check(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, const void* initial_state,
                         int initial_dtype, const void* d_out, const void* d_final_state,
                         int d_final_dtype, const int32_t* cu_seqlens, int32_t num_seqs,
                         int32_t B, int64_t T, int32_t H, int32_t K, int32_t V, const float* dq,
                         const float* dk, const float* dv, const float* dg, const float* dbeta,
                         const float* d_initial_state) {
  (void)scale;
  g_last_error.clear();
  return validate_bwd(q, k, v, g, beta, initial_state, initial_dtype, d_out, d_final_state,
                      d_final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, dq, dk, dv, dg, dbeta,
                      d_initial_state, nullptr);
}

int64_t kda_dim_workspace_bytes(int32_t n_sequences, int64_t rows, int32_t H, int32_t D) {
  if (n_sequences <= 0 || rows < 0 || H <= 0 || (D != 64 && D != 256)) return -1;
  if (rows == 0 || D == 64) return 0;
  return kda::dim_slots(n_sequences, rows) * H * (int64_t)kda::dim_record_bytes(D);
}

int64_t kda_bwd_workspace_bytes(int32_t n_sequences, int64_t rows, int32_t H) {
  if (n_sequences <= 0 || rows < 0 || H <= 0) return -1;
  return (int64_t)bwd_workspace_bytes(n_sequences, rows, H);
}

kda_status kda_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   float scale, const void* initial_state, int initial_dtype, const void* d_out,
                   const void* d_final_state, int d_final_dtype, const int32_t* cu_seqlens,
                   int32_t num_seqs, int32_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                   float* dq, float* dk, float* dv, float* dg, float* dbeta,
                   float* d_initial_state, void* stream) {
  g_last_error.clear();
  int32_t N = 0;
  kda_status st = validate_bwd(q, k, v, g, beta, initial_state, initial_dtype, d_out,
                               d_final_state, d_final_dtype, cu_seqlens, num_seqs, B, T, H, K, V,
                               dq, dk, dv, dg, dbeta, d_initial_state, &N);
  if (st != KDA_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t rows = cu_seqlens ? T : (int64_t)B * T;
  hipError_t e = hipSuccess;
  int cus = 0;
  if (device_cu_count(&cus) != 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count of the current device");
  const int64_t slots = bwd_slots(N, rows), gslots = bwd_group_slots(N, rows, H);
  const int64_t nb = gslots * H;   // batches of one group
  const BwdLayout lay = bwd_layout(N, rows, H);
  const size_t wbytes = lay.total;
  Workspace ws;
  e = ws.acquire(wbytes, hs);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "backward workspace of %zu bytes: %s", wbytes, hipGetErrorString(e));
  // carve one group's per-chunk tiles, then the checkpoints, the carries and the
  // forward pass's outputs
  kda::BwdTiles w{};
  char* const wbase = static_cast<char*>(ws.ptr());
  {
    float* base = reinterpret_cast<float*>(wbase);
    size_t off = 0;
    auto take = [&](size_t per) { float* r = base + off; off += (size_t)nb * per; return r; };
    float** t1[] = {&w.G, &w.kg, &w.qg, &w.kp, &w.vv, &w.dO,
                    &w.R, &w.U, &w.MtdO, &w.dU, &w.dY, &w.dqg, &w.dkg, &w.dkp};
    for (float** x : t1) *x = take(64 * 128);
    float** t2[] = {&w.A, &w.P, &w.M, &w.T, &w.dM, &w.dA};
    for (float** x : t2) *x = take(64 * 64);
    w.F = take(128 * 64);
    w.X = take(128 * 128);
    w.dSn = take(128 * 128);
    w.beta = take(64);
    w.gam = take(128);
    w.dgl = take(128);
    w.valid = reinterpret_cast<int*>(take(1));
    w.S = reinterpret_cast<float*>(wbase + lay.tiles);
  }
  float* carry = lay.carry ? reinterpret_cast<float*>(wbase + lay.tiles + lay.ckpt) : nullptr;
  uint16_t* fwd_out = reinterpret_cast<uint16_t*>(wbase + lay.tiles + lay.ckpt + lay.carry);
  hipError_t err = hipSuccess;
  if (rows > 0) {
    // forward pass with chunk checkpoints (no sequence splitting)
    kda::Params p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.g = g;
    p.beta = beta;
    p.out = fwd_out;
    p.s0 = initial_state;
    p.s0_fp32 = initial_dtype == KDA_FP32;
    p.cu = cu_seqlens;
    p.T = T;
    p.scale = scale;
    p.nseq = N;
    p.H = H;
    p.cus = cus;
    p.seg_min = seg_min_chunks();
    p.ckpt = w.S;
    p.dk = KDA_HEAD_DIM;
    const int nsplit = (int64_t)N * H >= cus ? 1 : 2;
    kda::BwdParams bp{};
    bp.q = p.q; bp.k = p.k; bp.v = p.v;
    bp.dout = static_cast<const uint16_t*>(d_out);
    bp.g = g; bp.beta = beta; bp.cu = cu_seqlens; bp.T = T; bp.scale = scale;
    bp.nseq = N; bp.H = H;
    bp.dsT = d_final_state; bp.dsT_fp32 = d_final_dtype == KDA_FP32;
    bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dg = dg; bp.dbeta = dbeta; bp.ds0 = d_initial_state;
    // the checkpointing forward pass and the products that need its checkpoints run
    // on a second stream of the library's, beside the work that does not
    hipStream_t side = nullptr;
    err = side_stream(&side);
    if (err == hipSuccess) err = kda::launch_bwd_streams(p, nsplit, bp, w, slots, gslots, carry, hs, side);
  } else if (d_initial_state != nullptr) {
    // no tokens: the initial-state gradient is the final-state gradient (or zero)
    kda::BwdParams bp{};
    bp.cu = cu_seqlens; bp.T = T; bp.nseq = N; bp.H = H;
    bp.dsT = d_final_state; bp.dsT_fp32 = d_final_dtype == KDA_FP32; bp.ds0 = d_initial_state;
    err = kda::launch_bwd_scan_only(bp, hs);
  }
  const hipError_t e2 = ws.release();
  if (err != hipSuccess) return fail(KDA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(err));
  if (e2 != hipSuccess) return fail(KDA_ERR_HIP, "workspace release: %s", hipGetErrorString(e2));
  return KDA_OK;
}

}  // extern "C"
