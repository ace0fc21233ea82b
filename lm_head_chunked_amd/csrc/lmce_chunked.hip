// The pages' own chunked formulation of the loss, natively on gfx950, as a
// comparison path for the fused kernels.
//
// Page: TRL docs "Training Beyond 1M Tokens", section "The massive logits
// matrix: chunk it": take a few hundred rows at a time (256 in TRL), form
// those rows' logits, compute their loss and add the pieces; the backward
// goes chunk by chunk the same way, each chunk adding its share to the
// weight gradient.  Here every chunk of chunk_rows rows:
//   forward   Z = h_c W^T            fp32 [rows][V] in the workspace (GEMM)
//             lse, nll of each row    (row kernel over Z)
//   backward  Z = h_c W^T            recomputed (GEMM)
//             G = g/N valid (softmax - onehot), bf16 (row kernel over Z,
//                 which also recomputes the row's lse)
//             dh_c = G W              (GEMM, K = V split over 16 pieces,
//                                      summed in a fixed order)
//             dW  += G^T h_c          (GEMM, first chunk stores)
// The L x V logits are never whole: at most one chunk's rows x V fp32 exist.

#include "lmce_device.h"
#include "lmce_internal.h"
#include "lmce.h"

namespace lmce {
namespace {

constexpr int kDhSplit = 16;  // K pieces of the dh GEMM (its output is only rows x H)

// Online (max, sum of exp) over one row held by a 256-thread workgroup;
// returns the row's log-sum-exp in every thread.
__device__ float row_lse(const float* __restrict__ z, int64_t V, float* red_m, float* red_s) {
  float m = -INFINITY, s = 0.f;
  for (int64_t v = threadIdx.x; v < V; v += 256) {
    const float x = z[v];
    if (x > m) {
      s = s * exp2_fast((m - x) * kLog2e) + 1.f;
      m = x;
    } else {
      s += exp2_fast((x - m) * kLog2e);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    const float M = fmaxf(m, m2);
    s = (M == -INFINITY) ? 0.f : s * exp2_fast((m - M) * kLog2e) + s2 * exp2_fast((m2 - M) * kLog2e);
    m = M;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_m[w] = m;
    red_s[w] = s;
  }
  __syncthreads();
  float M = red_m[0], S = red_s[0];
  for (int i = 1; i < 4; ++i) {
    const float mm = fmaxf(M, red_m[i]);
    S = S * exp2_fast((M - mm) * kLog2e) + red_s[i] * exp2_fast((red_m[i] - mm) * kLog2e);
    M = mm;
  }
  return M + logf(S);
}

// Forward row kernel: lse and nll of row r of the chunk (one workgroup per row).
__global__ __launch_bounds__(256) void k_chunk_lse(const float* __restrict__ Z, int64_t ldz, int64_t V,
                                                   const int64_t* __restrict__ labels, int64_t ignore_index,
                                                   float* __restrict__ lse_out, float* __restrict__ nll) {
  __shared__ float red_m[4], red_s[4];
  const int64_t r = blockIdx.x;
  const float* z = Z + r * ldz;
  const float lse = row_lse(z, V, red_m, red_s);
  if (threadIdx.x == 0) {
    const int64_t y = labels[r];
    const bool valid = y != ignore_index && y >= 0 && y < V;
    lse_out[r] = lse;
    nll[r] = valid ? lse - z[y] : 0.f;
  }
}

// Backward row kernel: G[r][v] = g/N * valid * (exp(z - lse) - [v == y]) in
// bf16 for v < V, 0 for V <= v < ldg (the K padding of the dh GEMM).
__global__ __launch_bounds__(256) void k_chunk_grad(const float* __restrict__ Z, int64_t ldz, int64_t V,
                                                    const int64_t* __restrict__ labels, int64_t ignore_index,
                                                    const float* __restrict__ grad_loss, const WsHeader* hdr,
                                                    uint16_t* __restrict__ G, int64_t ldg) {
  __shared__ float red_m[4], red_s[4];
  const int64_t r = blockIdx.x;
  const float* z = Z + r * ldz;
  const float lse = row_lse(z, V, red_m, red_s);
  const int64_t y = labels[r];
  const bool valid = y != ignore_index && y >= 0 && y < V;
  const int n = hdr->n_valid;
  const float scale = valid ? *grad_loss / (float)(n > 0 ? n : 1) : 0.f;
  const float l2 = lse * kLog2e;
  uint16_t* g = G + r * ldg;
  for (int64_t v = threadIdx.x; v < ldg; v += 256) {
    float x = 0.f;
    if (v < V) {
      const float pr = exp2_fast(__builtin_fmaf(z[v], kLog2e, -l2));
      x = scale * ((v == y) ? pr - 1.f : pr);
    }
    g[v] = __builtin_bit_cast(uint16_t, (__bf16)x);
  }
}

// dh row r = sum over the split pieces, in piece order.
__global__ __launch_bounds__(256) void k_chunk_dh_sum(const float* __restrict__ part, int64_t piece, int64_t H,
                                                      float* __restrict__ dh) {
  const int64_t r = blockIdx.x;
  for (int64_t c = threadIdx.x * 4; c < H; c += 1024) {
    float4 acc = *reinterpret_cast<const float4*>(part + r * H + c);
    for (int s = 1; s < kDhSplit; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(part + s * piece + r * H + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4*>(dh + r * H + c) = acc;
  }
}

// loss = sum of nll (fixed order: 1024 strided partial sums, then a tree) / N;
// NaN if N == 0 or this call saw a bad label.
__global__ __launch_bounds__(1024) void k_chunk_loss(const float* __restrict__ nll, int64_t L, const WsHeader* hdr,
                                                     float* __restrict__ loss_out) {
  __shared__ float red[1024];
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < L; i += 1024) acc += nll[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = hdr->n_valid;
    float loss = n > 0 ? red[0] / (float)n : __builtin_nanf("");
    if (hdr->call_flags != 0) loss = __builtin_nanf("");
    *loss_out = loss;
  }
}

constexpr int64_t kMaxRows = int64_t(1) << 21;

struct ChunkPlan {
  int64_t L, H, V, cr, Vg;
  size_t off_Z, off_G, off_part, off_nll, total;
};

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

int chunk_plan(int64_t L, int64_t H, int64_t V, int64_t chunk_rows, ChunkPlan* p) {
  if (L < 1 || L > kMaxRows || V < 1 || V > kMaxRows || H < 1 || H > 16384) return LMCE_ERR_SHAPE;
  if (H % 128 != 0 || chunk_rows < 1 || chunk_rows > 4096) return LMCE_ERR_UNSUPPORTED;
  p->L = L;
  p->H = H;
  p->V = V;
  p->cr = chunk_rows < L ? chunk_rows : L;
  p->Vg = (V + 128 * kDhSplit - 1) / (128 * kDhSplit) * (128 * kDhSplit);
  // the operands read MN-major (W over one dh piece of the vocabulary, G over
  // the chunk's rows) must fit one buffer resource, so that their 32-bit
  // offsets stay exact
  const int64_t kMaxRes = (int64_t)kMaxBufferBytes;
  const int64_t rk = (p->cr + 63) / 64 * 64;
  if ((p->Vg / kDhSplit + 1) * H * 2 > kMaxRes || rk * p->Vg * 2 > kMaxRes) return LMCE_ERR_UNSUPPORTED;
  size_t off = up256(sizeof(WsHeader));
  p->off_Z = off;
  off = up256(off + sizeof(float) * (size_t)p->cr * (size_t)p->Vg);
  p->off_G = off;
  off = up256(off + 2 * (size_t)p->cr * (size_t)p->Vg);
  p->off_part = off;
  off = up256(off + sizeof(float) * kDhSplit * (size_t)p->cr * (size_t)H);
  p->off_nll = off;
  off = up256(off + sizeof(float) * (size_t)L);
  p->total = off;
  return LMCE_OK;
}

bool aligned(const void* ptr, uintptr_t a) { return ptr != nullptr && (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Z = h_c W^T for the rows [r0, r0 + rows) into the workspace.
hipError_t chunk_logits(const ChunkPlan& p, const void* h, const void* W, int64_t r0, int64_t rows, void* ws,
                        hipStream_t s) {
  GemmArgs g = {};
  g.A = static_cast<const uint16_t*>(h) + r0 * p.H;
  g.a_bytes = (uint64_t)rows * p.H * 2;
  g.a_ld = (uint32_t)(p.H * 2);
  g.a_form = 0;
  g.B = W;
  g.b_bytes = (uint64_t)p.V * p.H * 2;
  g.b_ld = (uint32_t)(p.H * 2);
  g.b_form = 0;
  g.M = rows;
  g.N = p.V;
  g.kchunk = p.H;
  g.ksplit = 1;
  g.epi = kEpiStoreF32;
  g.alpha = 1.f;
  g.C = at(ws, p.off_Z);
  g.ldc = p.Vg;
  g.patch_m = 0;  // the tiles share only the chunk's h rows
  return launch_gemm(g, s);
}

}  // namespace
}  // namespace lmce

using namespace lmce;

extern "C" int lmce_chunked_workspace_size(int64_t L, int64_t H, int64_t V, int64_t chunk_rows, size_t* bytes) {
  if (bytes == nullptr) return LMCE_ERR_NULL;
  ChunkPlan p;
  const int st = chunk_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  *bytes = p.total;
  return LMCE_OK;
}

extern "C" int lmce_chunked_fwd(const void* h, const void* W, const int64_t* labels, int64_t L, int64_t H, int64_t V,
                                int64_t ignore_index, int64_t chunk_rows, float* loss_out, float* lse_out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  ChunkPlan p;
  int st = chunk_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(labels, 8) || !aligned(loss_out, 4) || !aligned(lse_out, 4) ||
      !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(workspace);
  if (launch_count_labels(labels, L, V, ignore_index, hdr, 0, s) != hipSuccess) return LMCE_ERR_HIP;
  float* nll = reinterpret_cast<float*>(at(workspace, p.off_nll));
  for (int64_t r0 = 0; r0 < L; r0 += p.cr) {
    const int64_t rows = (L - r0) < p.cr ? (L - r0) : p.cr;
    if (chunk_logits(p, h, W, r0, rows, workspace, s) != hipSuccess) return LMCE_ERR_HIP;
    hipLaunchKernelGGL(k_chunk_lse, dim3((unsigned)rows), dim3(256), 0, s,
                       reinterpret_cast<const float*>(at(workspace, p.off_Z)), p.Vg, V, labels + r0, ignore_index,
                       lse_out + r0, nll + r0);
    if (hipGetLastError() != hipSuccess) return LMCE_ERR_HIP;
  }
  hipLaunchKernelGGL(k_chunk_loss, dim3(1), dim3(1024), 0, s, (const float*)nll, L, (const WsHeader*)hdr, loss_out);
  return hipGetLastError() == hipSuccess ? LMCE_OK : LMCE_ERR_HIP;
}

extern "C" int lmce_chunked_bwd(const void* h, const void* W, const int64_t* labels, int64_t L, int64_t H, int64_t V,
                                int64_t ignore_index, int64_t chunk_rows, const float* grad_loss, float* dh_out,
                                float* dW_out, void* workspace, size_t workspace_bytes, void* stream) {
  ChunkPlan p;
  int st = chunk_plan(L, H, V, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(labels, 8) || !aligned(grad_loss, 4) || !aligned(dh_out, 16) ||
      !aligned(dW_out, 16) || !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(workspace);
  if (launch_count_labels(labels, L, V, ignore_index, hdr, -1, s) != hipSuccess) return LMCE_ERR_HIP;
  uint16_t* G = reinterpret_cast<uint16_t*>(at(workspace, p.off_G));
  float* part = reinterpret_cast<float*>(at(workspace, p.off_part));
  for (int64_t r0 = 0; r0 < L; r0 += p.cr) {
    const int64_t rows = (L - r0) < p.cr ? (L - r0) : p.cr;
    if (chunk_logits(p, h, W, r0, rows, workspace, s) != hipSuccess) return LMCE_ERR_HIP;
    hipLaunchKernelGGL(k_chunk_grad, dim3((unsigned)rows), dim3(256), 0, s,
                       reinterpret_cast<const float*>(at(workspace, p.off_Z)), p.Vg, V, labels + r0, ignore_index,
                       grad_loss, (const WsHeader*)hdr, G, p.Vg);
    if (hipGetLastError() != hipSuccess) return LMCE_ERR_HIP;
    // dh_c = G W: M = rows, N = H, K = Vg in kDhSplit pieces; W's rows are the
    // K index, read MN-major (rows past V read as zero)
    GemmArgs d = {};
    d.A = G;
    d.a_bytes = (uint64_t)rows * p.Vg * 2;
    d.a_ld = (uint32_t)(p.Vg * 2);
    d.a_form = 0;
    d.B = W;
    d.b_bytes = (uint64_t)V * H * 2;
    d.b_ld = (uint32_t)(H * 2);
    d.b_form = 2;
    d.M = rows;
    d.N = H;
    d.kchunk = p.Vg / kDhSplit;
    d.ksplit = kDhSplit;
    d.epi = kEpiStoreF32;
    d.alpha = 1.f;
    d.C = part;
    d.ldc = H;
    d.c_split = p.cr * H;
    d.patch_m = 0;  // few tiles: spread them over the XCDs
    if (launch_gemm(d, s) != hipSuccess) return LMCE_ERR_HIP;
    hipLaunchKernelGGL(k_chunk_dh_sum, dim3((unsigned)rows), dim3(256), 0, s, (const float*)part, p.cr * H, H,
                       dh_out + r0 * H);
    if (hipGetLastError() != hipSuccess) return LMCE_ERR_HIP;
    // dW += G^T h_c: M = V, N = H, K = the chunk's rows; G and the chunk's h
    // rows read MN-major (K rows past `rows` read as zero)
    GemmArgs w = {};
    w.A = G;
    w.a_bytes = (uint64_t)rows * p.Vg * 2;
    w.a_ld = (uint32_t)(p.Vg * 2);
    w.a_form = 2;
    w.B = static_cast<const uint16_t*>(h) + r0 * H;
    w.b_bytes = (uint64_t)rows * H * 2;
    w.b_ld = (uint32_t)(H * 2);
    w.b_form = 2;
    w.M = V;
    w.N = H;
    w.kchunk = (rows + 63) / 64 * 64;
    w.ksplit = 1;
    w.epi = r0 == 0 ? kEpiStoreF32 : kEpiAccF32;
    w.alpha = 1.f;
    w.C = dW_out;
    w.ldc = H;
    w.patch_m = 4;
    if (launch_gemm(w, s) != hipSuccess) return LMCE_ERR_HIP;
  }
  return LMCE_OK;
}
