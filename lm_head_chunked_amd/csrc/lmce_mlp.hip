// Sequence-tiled MLP block, forward and backward, on gfx950.
//
// Page: TRL docs "Training Beyond 1M Tokens", section "One GPU is not
// enough: split the sequence across many": one line of the model,
// down_proj(act_fn(gate_proj(x)) * up_proj(x)), builds four tensors at the
// full intermediate width I (4 x 19 GB at a million tokens and I = 9728).
// TRL PR #6845 lists MLP sequence tiling as the lever that removes them: the
// rows are processed a block at a time, so those tensors exist only for
// chunk_rows rows (in bf16, 2 bytes per element as on the page).  act_fn is
// SiLU.
//
// Weights: Wg, Wu [I][H] (gate_proj, up_proj), Wd [H][I] (down_proj), bf16.
// Per call the library packs Wg and Wu into one [2I][H] matrix whose rows
// alternate 32-row blocks of the two (rows 64q + j = Wg row 32q + j, rows
// 64q + 32 + j = Wu row 32q + j), so that one GEMM gives each lane the gate
// and up values of the same units.  Every other operand is read where it
// lies: the GEMM engine reads a row-major matrix either K-major or, for the
// contractions over the rows of another matrix, MN-major (transposing LDS
// reads), so no transposed copy is made.
//
// Forward, per chunk c:  p_c = silu(x_c Wg^T) * (x_c Wu^T)   (GEMM, fused epilogue, bf16)
//                        y_c = p_c Wd^T                      (GEMM, fp32 out)
// Backward, per chunk c (upstream dy):
//   gu_c = x_c [Wg; Wu]^T            recomputed (GEMM, bf16, fragment order)
//   dp_c = dy_c Wd (Wd read MN-major), and in the same epilogue dg_c, du_c and p_c (bf16, row-major)
//   dx_c = dg_c Wg + du_c Wu          (one GEMM over the packed 2I, read MN-major)
//   dWd += dy_c^T p_c, dWg += dg_c^T x_c, dWu += du_c^T x_c   (GEMMs over the chunk's rows, both
//                                                               operands read MN-major)
// Independent GEMMs share one grid (launch_gemm_group), so that their tiles
// pack the CUs instead of each leaving a partial last wave: in the forward
// chunk c's down GEMM with chunk c+1's gate/up GEMM (p alternates between two
// areas), in the backward dx_c with the three weight-gradient GEMMs.

#include "lmce_device.h"
#include "lmce_internal.h"
#include "lmce.h"

namespace lmce {
namespace {

// Packed gate/up rows (one 2I row per workgroup).
__global__ __launch_bounds__(256) void k_pack_gu(const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu,
                                                 int64_t H, uint16_t* __restrict__ Wgu) {
  const int64_t r = blockIdx.x;
  const int64_t q = r >> 6, j = r & 63;
  const uint16_t* src = (j < 32 ? Wg : Wu) + (q * 32 + (j & 31)) * H;
  const uint4* in = reinterpret_cast<const uint4*>(src);
  uint4* out = reinterpret_cast<uint4*>(Wgu + r * H);
  for (int64_t c = threadIdx.x; c < H / 8; c += 256) out[c] = in[c];
}

struct MlpPlan {
  int64_t L, H, I, cr;
  size_t off_Wgu, off_gu, off_act, off_dgu, total;
};

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

int mlp_plan(int64_t L, int64_t H, int64_t I, int64_t chunk_rows, MlpPlan* p) {
  if (L < 1 || L > (int64_t(1) << 24) || H < 128 || H > 16384 || I < 64 || I > 65536) return LMCE_ERR_SHAPE;
  if (H % 128 != 0 || I % 64 != 0 || chunk_rows < 1 || chunk_rows > 65536) return LMCE_ERR_UNSUPPORTED;
  p->L = L;
  p->H = H;
  p->I = I;
  p->cr = chunk_rows < L ? chunk_rows : L;
  // every operand read MN-major (the packed weights over K = 2I, Wd over
  // K = H, the chunk's rows over K = its rows) must fit one buffer resource,
  // so that its 32-bit offsets stay exact
  const int64_t kMaxRes = (int64_t)kMaxBufferBytes;
  const int64_t rp = (p->cr + 63) / 64 * 64;
  if (4 * I * H > kMaxRes || 4 * I * rp > kMaxRes) return LMCE_ERR_UNSUPPORTED;
  const size_t b = 2;  // bf16
  size_t off = up256(sizeof(WsHeader));
  p->off_Wgu = off;
  off = up256(off + b * 2 * I * H);
  p->off_gu = off;  // fragment order: whole 256 x 256 tiles
  off = up256(off + b * ((p->cr + 255) / 256 * 256) * ((2 * I + 255) / 256 * 256));
  p->off_act = off;
  off = up256(off + b * p->cr * I);
  p->off_dgu = off;
  off = up256(off + b * p->cr * 2 * I);
  p->total = off;
  return LMCE_OK;
}

bool aligned(const void* ptr, uintptr_t a) { return ptr != nullptr && (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// A K-major operand: `rows` rows of ld_elems bf16 each, K along a row.
void set_a_kmajor(GemmArgs& g, const void* p, int64_t rows, int64_t ld_elems) {
  g.A = p;
  g.a_bytes = (uint64_t)rows * ld_elems * 2;
  g.a_ld = (uint32_t)(ld_elems * 2);
  g.a_form = 0;
}
void set_b_kmajor(GemmArgs& g, const void* p, int64_t rows, int64_t ld_elems) {
  g.B = p;
  g.b_bytes = (uint64_t)rows * ld_elems * 2;
  g.b_ld = (uint32_t)(ld_elems * 2);
  g.b_form = 0;
}
// An MN-major operand: a row-major matrix of k_rows rows (the K index) and
// ld_elems columns (the operand's rows); K rows past k_rows read as zero.
void set_a_mnmajor(GemmArgs& g, const void* p, int64_t k_rows, int64_t ld_elems) {
  g.A = p;
  g.a_bytes = (uint64_t)k_rows * ld_elems * 2;
  g.a_ld = (uint32_t)(ld_elems * 2);
  g.a_form = 2;
}
void set_b_mnmajor(GemmArgs& g, const void* p, int64_t k_rows, int64_t ld_elems) {
  g.B = p;
  g.b_bytes = (uint64_t)k_rows * ld_elems * 2;
  g.b_ld = (uint32_t)(ld_elems * 2);
  g.b_form = 2;
}

// The gate/up GEMM of rows [r0, r0 + rows): p_c = silu(g) * u into `act`
// (rows x I, row-major); with store_gu, the bf16 gate/up values themselves
// into the gu area instead, in the GEMM's fragment order.
GemmArgs gate_up_args(const MlpPlan& p, const void* x, const uint16_t* Wgu, int64_t r0, int64_t rows, void* ws,
                      bool store_gu, uint16_t* act) {
  GemmArgs g = {};
  set_a_kmajor(g, static_cast<const uint16_t*>(x) + r0 * p.H, rows, p.H);
  set_b_kmajor(g, Wgu, 2 * p.I, p.H);
  g.M = rows;
  g.N = 2 * p.I;
  g.kchunk = p.H;
  g.ksplit = 1;
  g.alpha = 1.f;
  if (store_gu) {
    g.epi = kEpiStoreFrag;  // read back by the SwiGLU-backward epilogue, lane for lane
    g.C = at<uint16_t>(ws, p.off_gu);
  } else {
    g.epi = kEpiSwigluFwd;
    g.C = act;
    g.ldc = p.I;
  }
  g.patch_m = 4;
  return g;
}

// Packs Wg and Wu into the interleaved [2I][H] matrix.
hipError_t pack_weights(const MlpPlan& p, const void* Wg, const void* Wu, void* ws, hipStream_t s) {
  hipLaunchKernelGGL(k_pack_gu, dim3((unsigned)(2 * p.I)), dim3(256), 0, s, static_cast<const uint16_t*>(Wg),
                     static_cast<const uint16_t*>(Wu), p.H, at<uint16_t>(ws, p.off_Wgu));
  return hipGetLastError();
}

}  // namespace
}  // namespace lmce

using namespace lmce;

extern "C" int lmce_mlp_workspace_size(int64_t L, int64_t H, int64_t I, int64_t chunk_rows, size_t* bytes) {
  if (bytes == nullptr) return LMCE_ERR_NULL;
  MlpPlan p;
  const int st = mlp_plan(L, H, I, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  *bytes = p.total;
  return LMCE_OK;
}

extern "C" int lmce_mlp_fwd(const void* x, const void* Wg, const void* Wu, const void* Wd, int64_t L, int64_t H,
                            int64_t I, int64_t chunk_rows, float* y_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  MlpPlan p;
  int st = mlp_plan(L, H, I, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(x, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(y_out, 16) ||
      !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pack_weights(p, Wg, Wu, workspace, s) != hipSuccess) return LMCE_ERR_HIP;
  const uint16_t* Wgu = at<uint16_t>(workspace, p.off_Wgu);
  // p of consecutive chunks alternates between the act area and the gu area
  // (unused by the forward), so that each chunk's down GEMM runs in one grid
  // with the next chunk's gate/up GEMM
  uint16_t* const act_buf[2] = {at<uint16_t>(workspace, p.off_act), at<uint16_t>(workspace, p.off_gu)};
  int64_t rows0 = L < p.cr ? L : p.cr;
  if (launch_gemm(gate_up_args(p, x, Wgu, 0, rows0, workspace, false, act_buf[0]), s) != hipSuccess)
    return LMCE_ERR_HIP;
  for (int64_t r0 = 0, c = 0; r0 < L; r0 += p.cr, ++c) {
    const int64_t rows = (L - r0) < p.cr ? (L - r0) : p.cr;
    GemmArgs g[2] = {};
    set_a_kmajor(g[0], act_buf[c & 1], rows, I);
    set_b_kmajor(g[0], Wd, H, I);
    g[0].M = rows;
    g[0].N = H;
    g[0].kchunk = I;
    g[0].ksplit = 1;
    g[0].epi = kEpiStoreF32;
    g[0].alpha = 1.f;
    g[0].C = y_out + r0 * H;
    g[0].ldc = H;
    g[0].patch_m = 4;
    int n = 1;
    const int64_t r1 = r0 + p.cr;
    if (r1 < L) {
      const int64_t rows1 = (L - r1) < p.cr ? (L - r1) : p.cr;
      g[n++] = gate_up_args(p, x, Wgu, r1, rows1, workspace, false, act_buf[(c + 1) & 1]);
    }
    if (launch_gemm_group(g, n, s) != hipSuccess) return LMCE_ERR_HIP;
  }
  return LMCE_OK;
}

extern "C" int lmce_mlp_bwd(const void* x, const void* Wg, const void* Wu, const void* Wd, const void* dy, int64_t L,
                            int64_t H, int64_t I, int64_t chunk_rows, float* dx_out, float* dWg_out, float* dWu_out,
                            float* dWd_out, void* workspace, size_t workspace_bytes, void* stream) {
  MlpPlan p;
  int st = mlp_plan(L, H, I, chunk_rows, &p);
  if (st != LMCE_OK) return st;
  if (!aligned(x, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(dy, 16) ||
      !aligned(dx_out, 16) || !aligned(dWg_out, 16) || !aligned(dWu_out, 16) || !aligned(dWd_out, 16) ||
      !aligned(workspace, 256))
    return LMCE_ERR_NULL;
  if (workspace_bytes < p.total) return LMCE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pack_weights(p, Wg, Wu, workspace, s) != hipSuccess) return LMCE_ERR_HIP;
  // the weight gradients are sums over the chunks: start from zero (a fill
  // kernel, which graph capture records as an ordinary node)
  if (launch_zero_u32(reinterpret_cast<unsigned*>(dWg_out), (int)(I * H), s) != hipSuccess ||
      launch_zero_u32(reinterpret_cast<unsigned*>(dWu_out), (int)(I * H), s) != hipSuccess ||
      launch_zero_u32(reinterpret_cast<unsigned*>(dWd_out), (int)(H * I), s) != hipSuccess)
    return LMCE_ERR_HIP;
  const uint16_t* Wgu = at<uint16_t>(workspace, p.off_Wgu);
  uint16_t* gu = at<uint16_t>(workspace, p.off_gu);
  uint16_t* act = at<uint16_t>(workspace, p.off_act);
  uint16_t* dgu = at<uint16_t>(workspace, p.off_dgu);
  const uint16_t* x16 = static_cast<const uint16_t*>(x);
  const uint16_t* dy16 = static_cast<const uint16_t*>(dy);
  for (int64_t r0 = 0; r0 < L; r0 += p.cr) {
    const int64_t rows = (L - r0) < p.cr ? (L - r0) : p.cr;
    const int64_t rk = (rows + 63) / 64 * 64;  // K of the weight-gradient GEMMs (rows past `rows` read as zero)
    if (launch_gemm(gate_up_args(p, x, Wgu, r0, rows, workspace, true, nullptr), s) != hipSuccess)
      return LMCE_ERR_HIP;
    // dp = dy_c Wd (B = Wd read MN-major, K = H), epilogue: dg, du (packed like gu) and p
    GemmArgs d = {};
    set_a_kmajor(d, dy16 + r0 * H, rows, H);
    set_b_mnmajor(d, Wd, H, I);
    d.M = rows;
    d.N = I;
    d.kchunk = H;
    d.ksplit = 1;
    d.epi = kEpiSwigluBwd;
    d.alpha = 1.f;
    d.C = dgu;
    d.gu = gu;
    d.aux = act;
    d.patch_m = 4;
    if (launch_gemm(d, s) != hipSuccess) return LMCE_ERR_HIP;
    // dx_c = [dg | du] [Wg; Wu] (B = the packed matrix read MN-major, K = 2I)
    GemmArgs xg = {};
    set_a_kmajor(xg, dgu, rows, 2 * I);
    set_b_mnmajor(xg, Wgu, 2 * I, H);
    xg.M = rows;
    xg.N = H;
    xg.kchunk = 2 * I;
    xg.ksplit = 1;
    xg.epi = kEpiStoreF32;
    xg.alpha = 1.f;
    xg.C = dx_out + r0 * H;
    xg.ldc = H;
    xg.patch_m = 4;
    // weight gradients, K = the chunk's rows, both operands read MN-major
    GemmArgs wd = {};
    set_a_mnmajor(wd, dy16 + r0 * H, rows, H);
    set_b_mnmajor(wd, act, rows, I);
    wd.M = H;
    wd.N = I;
    wd.kchunk = rk;
    wd.ksplit = 1;
    wd.epi = kEpiAccF32;
    wd.alpha = 1.f;
    wd.C = dWd_out;
    wd.ldc = I;
    wd.patch_m = 4;
    GemmArgs wg = {};
    set_a_mnmajor(wg, dgu, rows, 2 * I);
    set_b_mnmajor(wg, x16 + r0 * H, rows, H);
    wg.M = 2 * I;
    wg.N = H;
    wg.kchunk = rk;
    wg.ksplit = 1;
    wg.epi = kEpiAccF32Gu;
    wg.alpha = 1.f;
    wg.C = dWg_out;
    wg.C2 = dWu_out;
    wg.ldc = H;
    wg.patch_m = 4;
    // the three are independent: one grid, the longest K first, so that their
    // tiles pack the CUs instead of each leaving a partial last wave (adding
    // the next chunk's gate/up recompute to the grid gained nothing)
    const GemmArgs three[3] = {xg, wg, wd};
    if (launch_gemm_group(three, 3, s) != hipSuccess) return LMCE_ERR_HIP;
  }
  return LMCE_OK;
}
