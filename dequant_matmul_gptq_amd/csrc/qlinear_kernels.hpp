// Host-side launchers of the gfx950 kernels. Arguments are validated by the
// C entry points before any of these is called.
#pragma once

#include "qlinear_device.hpp"

namespace qlinear {

Runs make_runs(const qlinear_layout& L);

hipError_t launch_pack(const qlinear_layout& L, const Runs& runs, const uint8_t* q, uint32_t* qweight,
                       hipStream_t stream);
hipError_t launch_unpack(const qlinear_layout& L, const Runs& runs, const uint32_t* qweight, uint8_t* q,
                         hipStream_t stream);
// scale_max non-NULL: scales holds two-level scale codes (uint32 [G][N/8]).
hipError_t launch_dequant(const qlinear_layout& L, const Runs& runs, const uint32_t* qweight,
                          const uint16_t* scales, const uint8_t* zeros, const uint16_t* scale_max, uint16_t* w,
                          hipStream_t stream);
// KV-cache codec over `elements` float16 values (rows of D, blocks of
// group in {32, 64, 128} elements, bits in {4, 6, 8}; elements % group == 0):
// codes uint32 [elements * bits / 32], scales float16 [elements / group].
hipError_t launch_kv_quant(const uint16_t* x, int64_t elements, int bits, int group, uint32_t* codes,
                           uint16_t* scales, hipStream_t stream);
hipError_t launch_kv_dequant(const uint32_t* codes, const uint16_t* scales, int64_t elements, int bits, int group,
                             uint16_t* x, hipStream_t stream);
// q_scale words [groups][N/8] from 4-bit codes [groups][N] (N % 8 == 0).
hipError_t launch_pack_qscale(const uint8_t* codes, int64_t groups, int64_t N, uint32_t* words,
                              hipStream_t stream);

// Act-order gather into unpacking pair order: xq uint32 [M][K/32][16] (float16
// pairs, optionally pre-scaled by 2^-pair_exponent), optional block sums
// xsum float2 [M][K/32] = (sum x, 1024 * sum of the scaled x).
// mfma: positions in MFMA pair order (mfma_pair), for the kernels that feed
// MFMA B fragments from the packed words.
hipError_t launch_gather_pairs(const Runs& runs, const uint16_t* x, const int32_t* perm, int M, int K,
                               uint32_t* xq, float2* xsum, bool scaled, bool mfma, hipStream_t stream);
// Prefill gather (no scaling, no sums): whole rows of x staged in LDS. Rows of
// more than kGatherRowsLds bytes use launch_gather_pairs.
constexpr size_t kGatherRowsLds = 64 * 1024;
hipError_t launch_gather_rows(const Runs& runs, const uint16_t* x, const int32_t* perm, int M, int K,
                              uint32_t* xq, bool mfma, hipStream_t stream);

// Decode layer (M <= 16). For M > 1 (and for rows too long for the fused
// M = 1 kernel) the workspace receives the gathered activations xq uint32
// [M][K/32][16] and the block sums xsum float2 [M][K/32]; it is scratch (no
// initialization, contents not preserved).
struct GemvWorkspace {
  uint32_t* xq;
  float2* xsum;
};
size_t qgemv_workspace_bytes(int K);
GemvWorkspace qgemv_workspace(void* ws, int K);
// mats (1 .. 8) matrices sharing the layout, x and perm: host arrays of
// their device pointers (zeros: NULL, or an array whose entries are all
// NULL or all not NULL).
hipError_t launch_qgemv(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M, const int32_t* perm,
                        int mats, const uint32_t* const* qweights, const uint16_t* const* scales,
                        const uint8_t* const* zeros, uint16_t* const* ys, void* ws, const Epilogue& epi,
                        hipStream_t stream);

// Prefill layer. ws holds the gathered activations, float16 [M][K].
// launch_qgemm_lds: the multiplication for layouts with several code widths,
// from activations already gathered (xq, float16 [M][K]).
// slices > 1 with part: K cut into that many slices whose float32 partial
// sums part[slices][M][N] are then added (split_sum_kernel).
hipError_t launch_qgemm_lds(const qlinear_layout& L, const Runs& runs, const uint16_t* xq, int M,
                            const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros, uint16_t* y,
                            const Epilogue& epi, int slices, float* part, hipStream_t stream);
// Decode layer on the matrix cores in factored form, 1 <= M <= 16, any set
// of code widths (qgemv_mx.hip). One launch with the act-order gather inside
// the kernel when qgemv_mx_one_launch() holds; otherwise a gather kernel
// writes the first qgemv_mx_workspace_bytes(K) bytes of the decode
// workspace (at most qgemv_workspace_bytes(K)) first. The packed words of a
// 64-column strip and the scales must each stay below 2^31 bytes
// (qgemv_mx_supported).
bool qgemv_mx_supported(const qlinear_layout& L);
bool qgemv_mx_one_launch(const qlinear_layout& L, int M, bool perm);
size_t qgemv_mx_workspace_bytes(int K);
hipError_t launch_qgemv_mx(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M,
                           const int32_t* perm, int mats, const uint32_t* const* qweights,
                           const uint16_t* const* scales, const uint8_t* const* zeros, uint16_t* const* ys,
                           void* ws, const Epilogue& epi, hipStream_t stream);

// Bytes of qgemm's workspace: the gathered activations [M][K] float16, then
// for layouts computed run by run the float32 partial sums [M][N].
size_t qgemm_workspace_bytes(const qlinear_layout& L, int M);
// Whether a call of M rows on a layout of several widths runs one launch per run.
bool qgemm_split_runs(const qlinear_layout& L, int M);
// Whether a call of M rows without two-level scales takes the LDS-dequant
// kernel, and into how many K slices that kernel cuts it.
bool qgemm_lds_path(const qlinear_layout& L, int M);
int qgemm_k_slices(const qlinear_layout& L, int M);
// Whether a prefill call of M rows runs as decode launches of 16 rows.
bool qgemm_as_decode(const qlinear_layout& L, int M);
// Whether the packed words and scales fit the prefill kernel's 32-bit offsets.
bool qgemm_supported(const qlinear_layout& L);
hipError_t launch_qgemm(const qlinear_layout& L, const Runs& runs, const uint16_t* x, int M,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        const int32_t* perm, uint16_t* y, void* ws, const Epilogue& epi, hipStream_t stream);

// On-the-fly LoRA update delta (+)= scale (x A) B. The workspace holds the
// partial sums of x A, float32 [lora_chunks(K)][M][rank].
int lora_chunks(int K);
size_t lora_workspace_bytes(int M, int K, int rank);
hipError_t launch_lora_delta(const uint16_t* x, int M, int K, const uint16_t* A, int rank, const uint16_t* B, int N,
                             float scale, bool accumulate, float* delta, void* ws, hipStream_t stream);

// Streaming-read floor (measurement helper): grid workgroups of 256 threads
// read `bytes` (a multiple of 16) with `loads` (4, 8 or 16) 16-byte loads in
// flight per thread.
hipError_t launch_read_floor(const void* buf, size_t bytes, int loads, int grid, uint32_t key, uint32_t* sink,
                             hipStream_t stream);

}  // namespace qlinear
