// extern "C" entry points of libqlinear: host-side validation, then launches
// on the caller's stream. Nothing here allocates memory or synchronizes.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "qlinear_kernels.hpp"

namespace qlinear {

Runs make_runs(const qlinear_layout& L) {
  Runs r;
  memset(&r, 0, sizeof(r));
  const int bpg = L.group_size / kBlockRows;
  r.nruns = L.nruns;
  r.blocks_per_group = bpg;
  r.packed_rows = L.packed_rows;
  for (int i = 0; i <= L.nruns; ++i) {
    r.run_block[i] = L.run_group[i] * bpg;
    r.run_row[i] = L.run_row[i];
  }
  for (int i = 0; i < L.nruns; ++i) r.run_bits[i] = L.run_bits[i];
  return r;
}

}  // namespace qlinear

namespace {

using namespace qlinear;

// Largest K accepted: the block count is a grid dimension (< 65536).
constexpr int64_t kMaxK = (int64_t)65535 * kBlockRows;
// Largest M of qlinear_qgemm: the several-width kernel takes row tiles of 128
// in one grid dimension.
constexpr int64_t kMaxGemmM = (int64_t)65535 * 128;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_bits(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }

// Structural check of a layout that the caller may have modified.
int check_layout(const qlinear_layout* L) {
  if (!L) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (L->K <= 0 || L->N <= 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (L->group_size != 32 && L->group_size != 64 && L->group_size != 128) return QLINEAR_ERR_UNSUPPORTED;
  if (L->K % L->group_size != 0 || L->N % 8 != 0 || L->K > kMaxK) return QLINEAR_ERR_UNSUPPORTED;
  if (L->groups != L->K / L->group_size) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (L->nruns < 1 || L->nruns > QLINEAR_MAX_RUNS) return QLINEAR_ERR_UNSUPPORTED;
  if (L->run_group[0] != 0 || L->run_row[0] != 0 || L->run_group[L->nruns] != L->groups)
    return QLINEAR_ERR_INVALID_ARGUMENT;
  const int bpg = L->group_size / kBlockRows;
  for (int r = 0; r < L->nruns; ++r) {
    if (!supported_bits(L->run_bits[r])) return QLINEAR_ERR_UNSUPPORTED;
    // Runs are maximal (qlinear_layout_init merges equal neighbours): the
    // launchers size workspaces and pick kernels from the run count.
    if (r > 0 && L->run_bits[r] == L->run_bits[r - 1]) return QLINEAR_ERR_INVALID_ARGUMENT;
    const int ng = L->run_group[r + 1] - L->run_group[r];
    if (ng <= 0) return QLINEAR_ERR_INVALID_ARGUMENT;
    if (L->run_row[r + 1] - L->run_row[r] != ng * bpg * L->run_bits[r]) return QLINEAR_ERR_INVALID_ARGUMENT;
  }
  if (L->run_row[L->nruns] != L->packed_rows) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (L->packed_words != (int64_t)((L->N + kPanel - 1) / kPanel) * L->packed_rows * kPanel)
    return QLINEAR_ERR_INVALID_ARGUMENT;
  return QLINEAR_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QLINEAR_OK : QLINEAR_ERR_HIP; }

int check_gemm_operands(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                        const uint16_t* scales, const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                        void* workspace) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (M < 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (M == 0) return QLINEAR_OK;  // quick return: no operand is touched (empty tensors may be NULL)
  if (!x || !qweight || !scales || !y) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!workspace) return QLINEAR_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y) || !aligned16(workspace) ||
      (zeros && !aligned16(zeros)) || (perm && !aligned16(perm)))
    return QLINEAR_ERR_MISALIGNED;
  return QLINEAR_OK;
}

// The epilogue of a fused call (NULL: none).
int check_epilogue(const qlinear_epilogue* e, Epilogue& out) {
  out = Epilogue{nullptr, nullptr, nullptr, QLINEAR_ACT_NONE, nullptr};
  if (!e) return QLINEAR_OK;
  if (e->activation != QLINEAR_ACT_NONE && e->activation != QLINEAR_ACT_SILU) return QLINEAR_ERR_UNSUPPORTED;
  if ((e->bias && !aligned16(e->bias)) || (e->residual && !aligned16(e->residual)) ||
      (e->addend && !aligned16(e->addend)))
    return QLINEAR_ERR_MISALIGNED;
  out = Epilogue{e->bias, e->residual, e->addend, e->activation, nullptr};
  return QLINEAR_OK;
}

// The two-level scale operands: q_scale (uint32 [G][N/8]) and q_scale_max
// (float16 [N]), both required; the epilogue then carries q_scale_max.
int check_qscale(const uint32_t* q_scale, const uint16_t* q_scale_max, Epilogue& epi) {
  if (!q_scale || !q_scale_max) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_scale) || !aligned16(q_scale_max)) return QLINEAR_ERR_MISALIGNED;
  epi.scale_max = q_scale_max;
  return QLINEAR_OK;
}

// Device scratch of qlinear_qgemv_noalloc: the decode workspace for any K up
// to QLINEAR_NOALLOC_MAX_K, held by every GPU the library runs on until the
// process ends. Zero at load; the decode kernels never need it cleared (they
// overwrite what they read). Host code never passes this name to a kernel:
// on the host it is only a stand-in for the symbol, and each device's
// address comes from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = (size_t)5 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The scratch address on the calling thread's current device, looked up once
// per device with that device current.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QLINEAR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QLINEAR_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return QLINEAR_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return QLINEAR_OK;
}

}  // namespace

extern "C" {

const char* qlinear_status_string(int status) {
  switch (status) {
    case QLINEAR_OK: return "ok";
    case QLINEAR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case QLINEAR_ERR_UNSUPPORTED: return "unsupported shape, group size, bit width or run count";
    case QLINEAR_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case QLINEAR_ERR_WORKSPACE: return "workspace missing or too small";
    case QLINEAR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int qlinear_group_order(const uint8_t* group_bits, int32_t groups, int32_t* order) {
  if (!group_bits || !order || groups <= 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  static const int kWidths[] = {8, 6, 5, 4, 3, 2};   // widest first
  for (int g = 0; g < groups; ++g) {
    const int b = group_bits[g];
    if (b != 2 && b != 3 && b != 4 && b != 5 && b != 6 && b != 8) return QLINEAR_ERR_UNSUPPORTED;
  }
  int n = 0;
  for (int b : kWidths)
    for (int g = 0; g < groups; ++g)
      if (group_bits[g] == b) order[n++] = g;
  return QLINEAR_OK;
}

int qlinear_layout_init(qlinear_layout* layout, int32_t K, int32_t N, int32_t group_size,
                        const uint8_t* bits_host) {
  if (!layout || !bits_host) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (K <= 0 || N <= 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (group_size != 32 && group_size != 64 && group_size != 128) return QLINEAR_ERR_UNSUPPORTED;
  if (K % group_size != 0 || N % 8 != 0 || K > kMaxK) return QLINEAR_ERR_UNSUPPORTED;
  qlinear_layout L;
  memset(&L, 0, sizeof(L));
  L.K = K;
  L.N = N;
  L.group_size = group_size;
  L.groups = K / group_size;
  const int bpg = group_size / kBlockRows;
  int nruns = 0;
  int64_t row = 0;
  for (int g = 0; g < L.groups; ++g) {
    const int b = bits_host[g];
    if (!supported_bits(b)) return QLINEAR_ERR_UNSUPPORTED;
    if (nruns == 0 || L.run_bits[nruns - 1] != b) {
      if (nruns == QLINEAR_MAX_RUNS) return QLINEAR_ERR_UNSUPPORTED;
      L.run_group[nruns] = g;
      L.run_row[nruns] = (int32_t)row;
      L.run_bits[nruns] = b;
      ++nruns;
    }
    row += (int64_t)bpg * b;
  }
  L.nruns = nruns;
  L.run_group[nruns] = L.groups;
  L.run_row[nruns] = (int32_t)row;
  L.packed_rows = (int32_t)row;
  L.packed_words = (int64_t)((N + kPanel - 1) / kPanel) * L.packed_rows * kPanel;
  *layout = L;
  return QLINEAR_OK;
}

int qlinear_pack_weights(const qlinear_layout* layout, const uint8_t* q, uint32_t* qweight, void* stream) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (!q || !qweight) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(qweight)) return QLINEAR_ERR_MISALIGNED;
  return hip_status(launch_pack(*layout, make_runs(*layout), q, qweight, (hipStream_t)stream));
}

int qlinear_unpack(const qlinear_layout* layout, const uint32_t* qweight, uint8_t* q, void* stream) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (!q || !qweight) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(qweight)) return QLINEAR_ERR_MISALIGNED;
  return hip_status(launch_unpack(*layout, make_runs(*layout), qweight, q, (hipStream_t)stream));
}

int qlinear_dequant(const qlinear_layout* layout, const uint32_t* qweight, const uint16_t* scales,
                    const uint8_t* zeros, uint16_t* w, void* stream) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (!qweight || !scales || !w) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(qweight) || !aligned16(scales) || !aligned16(w) || (zeros && !aligned16(zeros)))
    return QLINEAR_ERR_MISALIGNED;
  return hip_status(
      launch_dequant(*layout, make_runs(*layout), qweight, scales, zeros, nullptr, w, (hipStream_t)stream));
}

int qlinear_qgemv_workspace_bytes(const qlinear_layout* layout, size_t* bytes) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (!bytes) return QLINEAR_ERR_INVALID_ARGUMENT;
  *bytes = qgemv_workspace_bytes(layout->K);
  return QLINEAR_OK;
}

int qlinear_qgemv_fused(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                        const uint16_t* scales, const uint8_t* zeros, const int32_t* perm,
                        const qlinear_epilogue* epilogue, uint16_t* y, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_gemm_operands(layout, x, M, qweight, scales, zeros, perm, y, workspace);
  if (st != QLINEAR_OK) return st;
  Epilogue epi;
  st = check_epilogue(epilogue, epi);
  if (st != QLINEAR_OK || M == 0) return st;
  if (M > QLINEAR_GEMV_MAX_M || (M > 2 && !qgemv_mx_supported(*layout))) return QLINEAR_ERR_UNSUPPORTED;
  if (workspace_bytes < qgemv_workspace_bytes(layout->K)) return QLINEAR_ERR_WORKSPACE;
  return hip_status(launch_qgemv(*layout, make_runs(*layout), x, M, perm, 1, &qweight, &scales,
                                 zeros ? &zeros : nullptr, &y, workspace, epi, (hipStream_t)stream));
}

int qlinear_qgemv(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                  const uint16_t* scales, const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return qlinear_qgemv_fused(layout, x, M, qweight, scales, zeros, perm, nullptr, y, workspace, workspace_bytes,
                             stream);
}

int qlinear_qgemv_noalloc(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                          const uint16_t* scales, const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                          void* stream) {
  const int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (layout->K > QLINEAR_NOALLOC_MAX_K) return QLINEAR_ERR_UNSUPPORTED;
  if (M == 0) return QLINEAR_OK;
  const size_t need = qgemv_workspace_bytes(layout->K);
  if (need > kScratchBytes) return QLINEAR_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const int sst = scratch_on_current_device(&ws);
  if (sst != QLINEAR_OK) return sst;
  return qlinear_qgemv_fused(layout, x, M, qweight, scales, zeros, perm, nullptr, y, ws, need, stream);
}

int qlinear_qgemv_grouped(const qlinear_layout* layout, const uint16_t* x, int32_t M, int32_t count,
                          const uint32_t* const* qweights_host, const uint16_t* const* scales_host,
                          const uint8_t* const* zeros_host, const int32_t* perm, uint16_t* const* y_host,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (M < 0 || count < 1) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (count > QLINEAR_MAX_GROUP) return QLINEAR_ERR_UNSUPPORTED;
  if (!qweights_host || !scales_host || !y_host) return QLINEAR_ERR_INVALID_ARGUMENT;
  const bool zeros = zeros_host && zeros_host[0];
  for (int i = 0; i < count; ++i) {
    // every matrix is checked like the operands of qlinear_qgemv
    st = check_gemm_operands(layout, x, M, qweights_host[i], scales_host[i], zeros ? zeros_host[i] : nullptr, perm,
                             y_host[i], workspace);
    if (st != QLINEAR_OK) return st;
    if (zeros_host && (zeros_host[i] != nullptr) != zeros) return QLINEAR_ERR_INVALID_ARGUMENT;
  }
  if (M == 0) return QLINEAR_OK;
  if (M > QLINEAR_GEMV_MAX_M || (M > 2 && !qgemv_mx_supported(*layout))) return QLINEAR_ERR_UNSUPPORTED;
  if (workspace_bytes < qgemv_workspace_bytes(layout->K)) return QLINEAR_ERR_WORKSPACE;
  return hip_status(launch_qgemv(*layout, make_runs(*layout), x, M, perm, count, qweights_host, scales_host,
                                 zeros ? zeros_host : nullptr, y_host, workspace,
                                 Epilogue{nullptr, nullptr, nullptr, QLINEAR_ACT_NONE, nullptr},
                                 (hipStream_t)stream));
}

int qlinear_qgemm_workspace_bytes(const qlinear_layout* layout, int32_t M, size_t* bytes) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (!bytes || M < 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  *bytes = qgemm_workspace_bytes(*layout, M);
  return QLINEAR_OK;
}

int qlinear_qgemm_fused(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                        const uint16_t* scales, const uint8_t* zeros, const int32_t* perm,
                        const qlinear_epilogue* epilogue, uint16_t* y, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_gemm_operands(layout, x, M, qweight, scales, zeros, perm, y, workspace);
  if (st != QLINEAR_OK) return st;
  Epilogue epi;
  st = check_epilogue(epilogue, epi);
  if (st != QLINEAR_OK || M == 0) return st;
  if (M > kMaxGemmM || !qgemm_supported(*layout)) return QLINEAR_ERR_UNSUPPORTED;
  if (workspace_bytes < qgemm_workspace_bytes(*layout, M)) return QLINEAR_ERR_WORKSPACE;
  return hip_status(launch_qgemm(*layout, make_runs(*layout), x, M, qweight, scales, zeros, perm, y, workspace, epi,
                                 (hipStream_t)stream));
}

int qlinear_qgemm(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                  const uint16_t* scales, const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return qlinear_qgemm_fused(layout, x, M, qweight, scales, zeros, perm, nullptr, y, workspace, workspace_bytes,
                             stream);
}

int qlinear_pack_qscale(const uint8_t* codes, int32_t groups, int32_t N, uint32_t* q_scale, void* stream) {
  if (groups < 0 || N < 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (N % 8 != 0) return QLINEAR_ERR_UNSUPPORTED;
  if (groups == 0 || N == 0) return QLINEAR_OK;
  if (!codes || !q_scale) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(codes) || !aligned16(q_scale)) return QLINEAR_ERR_MISALIGNED;
  return hip_status(launch_pack_qscale(codes, groups, N, q_scale, (hipStream_t)stream));
}

int qlinear_dequant_qscale(const qlinear_layout* layout, const uint32_t* qweight, const uint32_t* q_scale,
                           const uint16_t* q_scale_max, uint16_t* w, void* stream) {
  int st = check_layout(layout);
  if (st != QLINEAR_OK) return st;
  if (!qweight || !w) return QLINEAR_ERR_INVALID_ARGUMENT;
  Epilogue epi{};
  st = check_qscale(q_scale, q_scale_max, epi);
  if (st != QLINEAR_OK) return st;
  if (!aligned16(qweight) || !aligned16(w)) return QLINEAR_ERR_MISALIGNED;
  return hip_status(launch_dequant(*layout, make_runs(*layout), qweight, reinterpret_cast<const uint16_t*>(q_scale),
                                   nullptr, q_scale_max, w, (hipStream_t)stream));
}

int qlinear_qgemv_qscale(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                         const uint32_t* q_scale, const uint16_t* q_scale_max, const int32_t* perm,
                         const qlinear_epilogue* epilogue, uint16_t* y, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(q_scale);
  int st = check_gemm_operands(layout, x, M, qweight, sc, nullptr, perm, y, workspace);
  if (st != QLINEAR_OK) return st;
  Epilogue epi;
  st = check_epilogue(epilogue, epi);
  if (st != QLINEAR_OK || M == 0) return st;
  st = check_qscale(q_scale, q_scale_max, epi);
  if (st != QLINEAR_OK) return st;
  if (M > QLINEAR_GEMV_MAX_M || (M > 2 && !qgemv_mx_supported(*layout))) return QLINEAR_ERR_UNSUPPORTED;
  if (workspace_bytes < qgemv_workspace_bytes(layout->K)) return QLINEAR_ERR_WORKSPACE;
  return hip_status(launch_qgemv(*layout, make_runs(*layout), x, M, perm, 1, &qweight, &sc, nullptr, &y, workspace,
                                 epi, (hipStream_t)stream));
}

int qlinear_qgemm_qscale(const qlinear_layout* layout, const uint16_t* x, int32_t M, const uint32_t* qweight,
                         const uint32_t* q_scale, const uint16_t* q_scale_max, const int32_t* perm,
                         const qlinear_epilogue* epilogue, uint16_t* y, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(q_scale);
  int st = check_gemm_operands(layout, x, M, qweight, sc, nullptr, perm, y, workspace);
  if (st != QLINEAR_OK) return st;
  Epilogue epi;
  st = check_epilogue(epilogue, epi);
  if (st != QLINEAR_OK || M == 0) return st;
  st = check_qscale(q_scale, q_scale_max, epi);
  if (st != QLINEAR_OK) return st;
  if (M > kMaxGemmM || !qgemm_supported(*layout)) return QLINEAR_ERR_UNSUPPORTED;
  if (workspace_bytes < qgemm_workspace_bytes(*layout, M)) return QLINEAR_ERR_WORKSPACE;
  return hip_status(launch_qgemm(*layout, make_runs(*layout), x, M, qweight, sc, nullptr, perm, y, workspace, epi,
                                 (hipStream_t)stream));
}

// The codec's shape and operand checks (shared by both directions).
static int check_kv(const void* x, int64_t rows, int32_t D, int32_t bits, int32_t group, const void* codes,
                    const void* scales) {
  if (rows < 0 || D <= 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (bits != 4 && bits != 6 && bits != 8) return QLINEAR_ERR_UNSUPPORTED;
  if ((group != 32 && group != 64 && group != 128) || D % group != 0) return QLINEAR_ERR_UNSUPPORTED;
  if (rows > ((int64_t)1 << 42) / D) return QLINEAR_ERR_UNSUPPORTED;
  if (rows == 0) return QLINEAR_OK;
  if (!x || !codes || !scales) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || ((uintptr_t)codes & 3u) || ((uintptr_t)scales & 1u)) return QLINEAR_ERR_MISALIGNED;
  return QLINEAR_OK;
}

int qlinear_kv_quant(const uint16_t* x, int64_t rows, int32_t D, int32_t bits, int32_t group, uint32_t* codes,
                     uint16_t* scales, void* stream) {
  const int st = check_kv(x, rows, D, bits, group, codes, scales);
  if (st != QLINEAR_OK || rows == 0) return st;
  return hip_status(launch_kv_quant(x, rows * D, bits, group, codes, scales, (hipStream_t)stream));
}

int qlinear_kv_dequant(const uint32_t* codes, const uint16_t* scales, int64_t rows, int32_t D, int32_t bits,
                       int32_t group, uint16_t* x, void* stream) {
  const int st = check_kv(x, rows, D, bits, group, codes, scales);
  if (st != QLINEAR_OK || rows == 0) return st;
  return hip_status(launch_kv_dequant(codes, scales, rows * D, bits, group, x, (hipStream_t)stream));
}

int qlinear_read_floor(const void* buf, size_t bytes, int32_t loads_per_thread, int32_t workgroups, uint32_t key,
                       uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (loads_per_thread != 4 && loads_per_thread != 8 && loads_per_thread != 16) return QLINEAR_ERR_UNSUPPORTED;
  if (workgroups < 1 || workgroups > 65535) return QLINEAR_ERR_UNSUPPORTED;
  if (!aligned16(buf) || !aligned16(sink)) return QLINEAR_ERR_MISALIGNED;
  return hip_status(launch_read_floor(buf, bytes, loads_per_thread, workgroups, key, sink, (hipStream_t)stream));
}

int qlinear_lora_workspace_bytes(int32_t M, int32_t K, int32_t rank, size_t* bytes) {
  if (!bytes || M < 0 || K < 1 || rank < 1) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (rank > QLINEAR_LORA_MAX_RANK || K > QLINEAR_LORA_MAX_DIM) return QLINEAR_ERR_UNSUPPORTED;
  *bytes = lora_workspace_bytes(M, K, rank);
  return QLINEAR_OK;
}

int qlinear_lora_delta(const uint16_t* x, int32_t M, int32_t K, const uint16_t* lora_a, int32_t rank,
                       const uint16_t* lora_b, int32_t N, float scale, int32_t accumulate, float* delta,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || K < 1 || N < 1 || rank < 1) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (rank > QLINEAR_LORA_MAX_RANK || K > QLINEAR_LORA_MAX_DIM || N > QLINEAR_LORA_MAX_DIM)
    return QLINEAR_ERR_UNSUPPORTED;
  if (M == 0) return QLINEAR_OK;
  if (!x || !lora_a || !lora_b || !delta) return QLINEAR_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < lora_workspace_bytes(M, K, rank)) return QLINEAR_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(lora_a) || !aligned16(lora_b) || !aligned16(delta) || !aligned16(workspace))
    return QLINEAR_ERR_MISALIGNED;
  return hip_status(launch_lora_delta(x, M, K, lora_a, rank, lora_b, N, scale, accumulate != 0, delta, workspace,
                                      (hipStream_t)stream));
}

}  // extern "C"
