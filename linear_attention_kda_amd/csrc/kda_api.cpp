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
                    const void* out, int32_t* n_out) {
  if (K != KDA_HEAD_DIM || V != KDA_HEAD_DIM)
    return fail(KDA_ERR_HEAD_DIM, "K=%d V=%d: only K = V = 128 is supported", K, V);
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
  const long double elems = (long double)B * (long double)T * (long double)H * KDA_HEAD_DIM;
  if (elems > (long double)(INT64_MAX / 4))
    return fail(KDA_ERR_SHAPE, "tensor size overflows 64-bit indexing");
  if ((int64_t)N * H * 2 > (int64_t)INT_MAX - 64)
    return fail(KDA_ERR_SHAPE, "N*H=%lld too large", (long long)N * H);
  if (T > 0) {
    if (!q || !k || !v || !g || !beta || !out)
      return fail(KDA_ERR_NULL, "q, k, v, g, beta and out are required when T > 0");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) ||
        !aligned(out, 16))
      return fail(KDA_ERR_ALIGN, "q, k, v, g and out must be 16-byte aligned");
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

int choose_splits(int32_t N, int32_t H, int32_t cus) {
  const char* e = std::getenv("KDA_VSPLIT");
  if (e != nullptr && (e[0] == '1' || e[0] == '2') && e[1] == '\0') return e[0] - '0';
  // one workgroup per (sequence, head) already covers the CUs: no value split
  return ((int64_t)N * H >= cus) ? 1 : 2;
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "required pointer is NULL";
    case KDA_ERR_HEAD_DIM: return "head dimension must be 128";
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
                  cu_seqlens, num_seqs, B, T, H, K, V, out, nullptr);
}

kda_status kda_plan(int32_t n_sequences, int32_t H, int32_t cu_count, int32_t* workgroups,
                    int32_t* value_splits) {
  g_last_error.clear();
  if (!workgroups || !value_splits) return fail(KDA_ERR_NULL, "kda_plan outputs are NULL");
  if (n_sequences <= 0 || H <= 0)
    return fail(KDA_ERR_SHAPE, "kda_plan: N=%d H=%d", n_sequences, H);
  int cus = cu_count;
  if (cus <= 0 && device_cu_count(&cus) != 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count of the current device");
  const int ns = choose_splits(n_sequences, H, cus);
  const int64_t pairs = (int64_t)n_sequences * H;
  *value_splits = ns;
  *workgroups = (int32_t)(((pairs + 7) / 8) * 8 * ns);
  return KDA_OK;
}

kda_status kda_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   float scale, const void* initial_state, int initial_dtype, void* final_state,
                   int final_dtype, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                   int64_t T, int32_t H, int32_t K, int32_t V, void* out, void* stream) {
  g_last_error.clear();
  int32_t N = 0;
  kda_status st = validate(q, k, v, g, beta, initial_state, initial_dtype, final_state,
                           final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out, &N);
  if (st != KDA_OK) return st;
  if (T == 0 && final_state == nullptr) return KDA_OK;  // nothing observable to compute

  int cus = 0;
  if (device_cu_count(&cus) != 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count of the current device");
  const int ns = choose_splits(N, H, cus);

  kda::Params p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = g;
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
  if (log_enabled())
    std::fprintf(stderr, "[kda] launch: N=%d H=%d T=%lld value_splits=%d cus=%d varlen=%d\n", N,
                 H, (long long)T, ns, cus, cu_seqlens != nullptr);
  const hipError_t err = kda::launch_fwd(p, ns, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return KDA_OK;
}

}  // extern "C"
