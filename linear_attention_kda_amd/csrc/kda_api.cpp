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
#include <mutex>
#include <string>

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

// The device's segment plan for N equal sequences of c chunks (fixed-length
// batches): does it split them?  Same rule as the kernels' plan.
bool fixed_length_splits(int64_t N, int64_t c, int64_t H, int64_t cus, int seg_min, int emax) {
  if (c <= seg_min) return false;
  auto fits = [&](int64_t m) {
    return kda::kSlackDen * H * (N * c + N * (c > m ? c - m : 0)) <= kda::kSlackNum * m * cus;
  };
  if (!fits(c)) return false;
  int64_t lo = seg_min, hi = c;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (fits(mid)) hi = mid;
    else lo = mid + 1;
  }
  return hi < c && N * ((c + hi - 1) / hi - 1) <= emax;
}

struct LaunchPlan {
  int nsplit;     // value-column slices per (sequence, head)
  int emax;       // segment state slots (0: no sequence splitting)
  int seg_min;
  int64_t workgroups;
  size_t workspace;
};

// rows: packed rows (T with cu_seqlens, else B*T); T: tokens per row, or the
// packed total with cu_seqlens.
LaunchPlan make_plan(int32_t N, int64_t T, int32_t H, bool varlen, int32_t cus) {
  LaunchPlan lp{};
  lp.seg_min = seg_min_chunks();
  const int forced = forced_splits();
  const int64_t c_max = (T + KDA_CHUNK - 1) / KDA_CHUNK;  // chunks of the longest possible sequence
  int emax = 0;
  // the device plan counts chunks and fix-up units in 32-bit integers
  const int64_t chunks = (varlen ? c_max + N : (int64_t)N * c_max);
  const bool small_enough = chunks < (1LL << 30) && chunks * H < (1LL << 30);
  if (seq_split_enabled() && forced != 2 && N <= kda::kSortLimit && c_max > lp.seg_min &&
      small_enough) {
    emax = kda::workspace_slots(cus, H);
    if (emax > 512) emax = 512;
    if (emax > 0 && !varlen && !fixed_length_splits(N, c_max, H, cus, lp.seg_min, emax)) emax = 0;
  }
  lp.emax = emax;
  // one workgroup per (sequence, head) already covers the CUs: no value split
  lp.nsplit = forced ? forced : (emax > 0 || (int64_t)N * H >= cus) ? 1 : 2;
  if (emax > 0 && lp.nsplit != 1) lp.emax = emax = 0;
  const int64_t groups = (int64_t)N + (emax > 0 ? 2 * (int64_t)emax : 0);
  lp.workgroups = (groups * H + 7) / 8 * 8 * lp.nsplit;
  const int64_t rows = varlen ? T : (int64_t)N * T;
  lp.workspace = emax > 0 ? kda::workspace_layout(rows, H, emax).total : 0;
  return lp;
}

// Library-owned stream-ordered pool for the splitting workspace, one per device.
// It keeps what it has reserved (release threshold at maximum), so after the
// first call of a given size a workspace costs no allocation from the driver.
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
    uint64_t keep = UINT64_MAX;
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

// Head dimensions 64 and 256: per-chunk records in a workspace from the pool,
// then the serial state pass (no sequence splitting).
kda_status fwd_dim_impl(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, float scale, const void* initial_state,
                        int initial_dtype, void* final_state, int final_dtype,
                        const int32_t* cu_seqlens, int32_t N, int32_t B, int64_t T, int32_t H,
                        int32_t D, void* out, void* stream, bool g_scalar) {
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
  void* ws = nullptr;
  if (bytes > 0) {
    hipMemPool_t pool = nullptr;
    hipError_t e = workspace_pool(&pool);
    if (e == hipSuccess) e = hipMallocFromPoolAsync(&ws, bytes, pool, hs);
    if (e != hipSuccess)
      return fail(KDA_ERR_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    p.ws = static_cast<char*>(ws);
  }
  if (log_enabled())
    std::fprintf(stderr, "[kda] launch: %s D=%d N=%d H=%d T=%lld record_slots=%lld workspace=%zu\n",
                 g_scalar ? "gdn" : "kda", D, N, H, (long long)T, (long long)p.slots, bytes);
  const hipError_t err = kda::launch_fwd_dim(p, hs);
  if (ws != nullptr) {
    const hipError_t e = hipFreeAsync(ws, hs);
    if (err == hipSuccess && e != hipSuccess)
      return fail(KDA_ERR_HIP, "workspace release: %s", hipGetErrorString(e));
  }
  if (err != hipSuccess)
    return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return KDA_OK;
}

kda_status fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    float scale, const void* initial_state, int initial_dtype, void* final_state,
                    int final_dtype, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                    int64_t T, int32_t H, int32_t K, int32_t V, void* out, void* stream,
                    bool g_scalar) {
  g_last_error.clear();
  int32_t N = 0;
  kda_status st = validate(q, k, v, g, beta, initial_state, initial_dtype, final_state,
                           final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out, &N,
                           g_scalar);
  if (st != KDA_OK) return st;
  if (T == 0 && final_state == nullptr) return KDA_OK;  // nothing observable to compute
  if (K != KDA_HEAD_DIM)
    return fwd_dim_impl(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state,
                        final_dtype, cu_seqlens, N, B, T, H, K, out, stream, g_scalar);

  int cus = 0;
  if (device_cu_count(&cus) != 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count of the current device");
  const LaunchPlan lp = make_plan(N, T, H, cu_seqlens != nullptr, cus);
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
  p.cus = cus;
  p.seg_min = lp.seg_min;
  void* ws = nullptr;
  if (lp.emax > 0) {
    hipMemPool_t pool = nullptr;
    hipError_t e = workspace_pool(&pool);
    if (e == hipSuccess) e = hipMallocFromPoolAsync(&ws, lp.workspace, pool, hs);
    if (e != hipSuccess)
      return fail(KDA_ERR_HIP, "workspace of %zu bytes: %s", lp.workspace, hipGetErrorString(e));
    const kda::WorkspaceLayout wl =
        kda::workspace_layout(cu_seqlens ? T : (int64_t)B * T, H, lp.emax);
    p.emax = lp.emax;
    p.o0 = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + wl.o0);
    p.st = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.st);
    p.sb = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + wl.sb);
  }
  if (log_enabled())
    std::fprintf(stderr,
                 "[kda] launch: %s N=%d H=%d T=%lld value_splits=%d cus=%d varlen=%d "
                 "segment_slots=%d workspace=%zu\n",
                 g_scalar ? "gdn" : "kda", N, H, (long long)T, lp.nsplit, cus,
                 cu_seqlens != nullptr, lp.emax, lp.workspace);
  const hipError_t err = kda::launch_fwd(p, lp.nsplit, hs);
  if (ws != nullptr) {
    const hipError_t e = hipFreeAsync(ws, hs);
    if (err == hipSuccess && e != hipSuccess)
      return fail(KDA_ERR_HIP, "workspace release: %s", hipGetErrorString(e));
  }
  if (err != hipSuccess)
    return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return KDA_OK;
}

}  // namespace

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
    default: return "unknown status";
  }
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

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
  return fwd_impl(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state, final_dtype,
                  cu_seqlens, num_seqs, B, T, H, K, V, out, stream, false);
}

kda_status kda_gdn_fwd(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float scale, const void* initial_state,
                       int initial_dtype, void* final_state, int final_dtype,
                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                       int32_t H, int32_t K, int32_t V, void* out, void* stream) {
  return fwd_impl(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state, final_dtype,
                  cu_seqlens, num_seqs, B, T, H, K, V, out, stream, true);
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

size_t bwd_workspace_bytes(int32_t N, int64_t rows, int32_t H) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nb = (size_t)bwd_slots(N, rows) * H;
  return up(nb * kda::BwdTiles::floats_per_batch() * 4) + up((size_t)rows * H * 128 * 2);
}

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
  if (rows == 0) return 0;
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
  const size_t gbytes = (size_t)rows * H * 128 * 4;
  hipError_t e = hipSuccess;
  // rows outside every sequence get zero gradients
  if (rows > 0) {
    e = hipMemsetAsync(dq, 0, gbytes, hs);
    if (e == hipSuccess) e = hipMemsetAsync(dk, 0, gbytes, hs);
    if (e == hipSuccess) e = hipMemsetAsync(dv, 0, gbytes, hs);
    if (e == hipSuccess) e = hipMemsetAsync(dg, 0, gbytes, hs);
    if (e == hipSuccess) e = hipMemsetAsync(dbeta, 0, (size_t)rows * H * 4, hs);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "gradient clear: %s", hipGetErrorString(e));
  }
  int cus = 0;
  if (device_cu_count(&cus) != 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count of the current device");
  const int64_t nb = bwd_slots(N, rows) * H;
  const size_t wbytes = bwd_workspace_bytes(N, rows, H);
  hipMemPool_t pool = nullptr;
  void* ws = nullptr;
  e = workspace_pool(&pool);
  if (e == hipSuccess) e = hipMallocFromPoolAsync(&ws, wbytes, pool, hs);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "backward workspace of %zu bytes: %s", wbytes, hipGetErrorString(e));
  // carve the per-chunk tiles
  kda::BwdTiles w{};
  {
    float* base = static_cast<float*>(ws);
    size_t off = 0;
    auto take = [&](size_t per) { float* r = base + off; off += (size_t)nb * per; return r; };
    float** t1[] = {&w.G, &w.kg, &w.qg, &w.kh, &w.kp, &w.vv, &w.dO,
                    &w.R, &w.U, &w.MtdO, &w.dU, &w.dY, &w.dqg, &w.dkg, &w.dkh, &w.dkp};
    for (float** x : t1) *x = take(64 * 128);
    float** t2[] = {&w.A, &w.P, &w.M, &w.T, &w.dM, &w.dA};
    for (float** x : t2) *x = take(64 * 64);
    w.F = take(128 * 64);
    w.S = take(128 * 128);
    w.X = take(128 * 128);
    w.dSn = take(128 * 128);
    w.beta = take(64);
    w.gam = take(128);
    w.valid = reinterpret_cast<int*>(take(1));
  }
  uint16_t* fwd_out = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) +
                                                   ((nb * kda::BwdTiles::floats_per_batch() * 4 + 255) & ~(size_t)255));
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
    const int nsplit = (int64_t)N * H >= cus ? 1 : 2;
    err = kda::launch_fwd(p, nsplit, hs);
    if (err == hipSuccess) {
      kda::BwdParams bp{};
      bp.q = p.q; bp.k = p.k; bp.v = p.v;
      bp.dout = static_cast<const uint16_t*>(d_out);
      bp.g = g; bp.beta = beta; bp.cu = cu_seqlens; bp.T = T; bp.scale = scale;
      bp.nseq = N; bp.H = H;
      bp.dsT = d_final_state; bp.dsT_fp32 = d_final_dtype == KDA_FP32;
      bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dg = dg; bp.dbeta = dbeta; bp.ds0 = d_initial_state;
      err = kda::launch_bwd(bp, w, nb, hs);
    }
  } else if (d_initial_state != nullptr) {
    // no tokens: the initial-state gradient is the final-state gradient (or zero)
    kda::BwdParams bp{};
    bp.cu = cu_seqlens; bp.T = T; bp.nseq = N; bp.H = H;
    bp.dsT = d_final_state; bp.dsT_fp32 = d_final_dtype == KDA_FP32; bp.ds0 = d_initial_state;
    err = kda::launch_bwd_scan_only(bp, hs);
  }
  const hipError_t e2 = hipFreeAsync(ws, hs);
  if (err != hipSuccess) return fail(KDA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(err));
  if (e2 != hipSuccess) return fail(KDA_ERR_HIP, "workspace release: %s", hipGetErrorString(e2));
  return KDA_OK;
}

}  // extern "C"
