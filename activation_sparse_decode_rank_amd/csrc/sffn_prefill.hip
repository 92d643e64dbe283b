// Dense prefill on the matrix cores (gfx950): the FFN over every neuron for many tokens at
// once, which the pages run dense (PowerInfer-2 article, section 4.1.1 NPU-Centric Prefill:
// prefill takes the whole layer, no activation prediction). At hundreds of tokens the two
// products are dense matrix products, so they are blocked for reuse: each weight tile is
// read once per 128 tokens instead of once per 64-token chunk of the decode kernels.
//
// Arithmetic as on the decode path's matrix-core kernels: fp16 weights as stored, fp32
// activations carried as fp16 hi + lo pairs (two products each, about 22 significant bits),
// v_mfma_f32_16x16x32_f16 with fp32 accumulation. The kernels' LO = false form (asked for
// with SFFN_PREFILL_FP16_ACT) rounds the activations (x and h) to fp16 once and runs one
// product each, half the matrix-core work and operand traffic, at fp16 activation precision.
//
// The kernels of a chunk of Bp tokens (Bp a multiple of 128; rows past the chunk's tokens
// are zero):
//  - k_pf_split: x [B][d] fp32 -> xh, xl [Bp][d] fp16;
//  - k_pf_up:    h = relu(W_act x + b_act) (gated: times W_up x) for every neuron and token,
//                as hh, hl [Bp][np] fp16 (np = d_ffn rounded up to the neuron tile, 64 to
//                192; neurons past d_ffn are 0);
//  - k_pf_down:  y = h W_down^T + b_out, the neurons split S ways (S a power of 2 up to
//                16) when the output tiles alone do not fill the GPU; the S partial sums go
//                to scratch and k_pf_sum adds them in split order (y bitwise reproducible).
// Both products stream their operands from memory straight into LDS through a pipeline of
// several stages; the down kernel reads W_down's rows there with the LDS transpose read.
#include "sffn_device.h"
#include "sffn_host.h"

namespace sffn {
namespace {

constexpr int PF_T = host::kPfTile;  // tokens per tile, and output columns per down tile
// s_waitcnt operand (gfx9 encoding) that waits for LDS reads only: lgkmcnt 0, vmcnt and
// expcnt at their maximum
constexpr int WAIT_LGKM0 = 0xC07F;

__device__ __forceinline__ float4_t pf_mfma(const half8_t& a, const half8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// x [B][d] fp32 -> hi, lo [Bp][d] fp16 (LO: lo as well), rows B .. Bp-1 zero
template <bool LO>
__global__ __launch_bounds__(TPB) void k_pf_split(const float* __restrict__ x, int B, int Bp, int d,
                                                  u32x4* __restrict__ xh, u32x4* __restrict__ xl) {
  const int nch = d / 8;
  const size_t total = (size_t)Bp * nch;
  for (size_t q = (size_t)blockIdx.x * TPB + threadIdx.x; q < total; q += (size_t)gridDim.x * TPB) {
    const int b = (int)(q / nch), c = (int)(q % nch);
    float4_t a = {0.f, 0.f, 0.f, 0.f}, e = {0.f, 0.f, 0.f, 0.f};
    if (b < B) {
      const float4_t* p = reinterpret_cast<const float4_t*>(x + (size_t)b * d + (size_t)c * 8);
      a = p[0];
      e = p[1];
    }
    half8_t hi, lo;
    split_hi_lo(a, e, hi, lo);
    xh[q] = __builtin_bit_cast(u32x4, hi);
    if (LO) xl[q] = __builtin_bit_cast(u32x4, lo);
  }
}

// Up projection: workgroup (mt, bt) computes neurons [MR mt, +MR) x tokens [128 bt, +128)
// (MR = 32 IT: 64, 96, 128 or 192) over all d inputs, in stages of 32 inputs. Wave w takes
// neurons 16 IT (w & 1) .. +16 IT and tokens 64 (w >> 1) .. +64 (IT x 4 tiles of 16 x 16,
// for the gate and, gated, the up matrix). The operands reach LDS without passing through
// registers (global_load_lds_dwordx4: each lane's 16 bytes land at the next 16 bytes of a
// 1 KB block), NS stages deep. A stage holds, per operand (each weight matrix, the tokens'
// hi and lo halves), its rows x 64 bytes; within each 16-row group, row r's 16-byte chunk c
// sits at position (c + r / 4) mod 4 of the row, so that a fragment read (16 rows, one
// chunk each) touches every LDS bank once. Each step waits for the next stage, refills the
// buffer just read with the stage NS ahead, and reads the next stage's fragments into
// registers while the matrix cores take the current ones; two fragment sets alternate, so
// the loop runs two steps a turn. Neuron tiles mt of the same bt are 8 apart in the grid
// when the neuron tile count is padded to a multiple of 8, so the workgroups sharing a
// weight tile run on one XCD.
constexpr int PFD_K = 32;  // inputs per stage
template <bool GATED, int IT, bool LO>
__global__ __launch_bounds__(TPB) void k_pf_up(const void* __restrict__ w_act, int ld_act,
                                               const float* __restrict__ b_act,
                                               const u32x4* __restrict__ xh,
                                               const u32x4* __restrict__ xl, int d, int n,
                                               int np, int nmt, _Float16* __restrict__ hh,
                                               _Float16* __restrict__ hl) {
  constexpr int NM = GATED ? 2 : 1;
  constexpr int MR = 32 * IT;                  // neurons per workgroup
  constexpr int GA = MR / 16, GB = PF_T / 16;  // 16-row groups of a weight / token operand
  constexpr int BLK_A = MR * PFD_K, BLK_B = PF_T * PFD_K;  // halfs per operand block
  constexpr int NB = LO ? 2 : 1;                           // token blocks (hi, lo)
  constexpr int STAGE = NM * BLK_A + NB * BLK_B;           // halfs per stage
  // stages held in LDS: tiles of up to 96 neurons keep two workgroups a compute unit (80 KB
  // each), the larger tiles one (up to 128 KB)
  constexpr int NS = IT <= 3 ? ((80 * 1024) / (STAGE * 2) < 4 ? (80 * 1024) / (STAGE * 2) : 4)
                             : (STAGE * 2 * 4 <= 128 * 1024 ? 4 : 3);
  constexpr int NG = NM * GA + NB * GB;                    // 1 KB loads a stage
  constexpr int DPS = NG / (TPB / 64);                     // load instructions per wave a stage
  static_assert(NG % (TPB / 64) == 0, "whole loads per wave");
  __shared__ __attribute__((aligned(16))) _Float16 sbuf[NS * STAGE];
  const int nmt_pad = (nmt + 7) / 8 * 8;
  const int mt = blockIdx.x % nmt_pad, bt = blockIdx.x / nmt_pad;
  if (mt >= nmt) return;  // padding workgroup (uniform)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int nch = d / 8;
  const int m0 = mt * MR, b0 = bt * PF_T;
  const u32x4* w = static_cast<const u32x4*>(w_act);
  const int nk = d / PFD_K;

  // the lane's row in a 16-row group and the global chunk its LDS position holds
  const int lr = lane >> 2;
  const int lc = ((lane & 3) - (lr >> 2)) & 3;
  auto issue = [&](int st, int buf) {
    const int kc = st * (PFD_K / 8) + lc;
    _Float16* base = sbuf + buf * STAGE;
#pragma unroll
    for (int v = 0; v < DPS; ++v) {
      const int u = wave + (TPB / 64) * v;  // 16-row group of some operand, wave-uniform
      const u32x4* src;
      int off;
      if (u < NM * GA) {
        const int o = u / GA, q = u % GA;
        src = w + (size_t)min(m0 + q * 16 + lr, n - 1) * ld_act + (size_t)o * nch + kc;
        off = o * BLK_A + q * 16 * PFD_K;
      } else {
        const int o = (u - NM * GA) / GB, q = (u - NM * GA) % GB;
        src = (o == 0 ? xh : xl) + (size_t)(b0 + q * 16 + lr) * nch + kc;
        off = NM * BLK_A + o * BLK_B + q * 16 * PFD_K;
      }
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(base + off),
                                       16, 0, 0);
    }
  };
  // fragment read: rows R .. R + 15 (R a multiple of 16) of the block at off, chunk g
  auto frag = [&](const _Float16* base, int off, int R) {
    return *reinterpret_cast<const half8_t*>(
        base + off + R * PFD_K + (r16 * 4 + ((g + (r16 >> 2)) & 3)) * 8);
  };
  float4_t acc[NM][IT][4];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[m][i][t] = float4_t{0.f, 0.f, 0.f, 0.f};

  struct Frags {
    half8_t b[NB][4];
    half8_t a[NM][IT];
  };
  auto read_frags = [&](Frags& F, int st) {
    const _Float16* base = sbuf + (st % NS) * STAGE;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      F.b[0][t] = frag(base, NM * BLK_A, wn * 64 + t * 16);
      if constexpr (LO) F.b[NB - 1][t] = frag(base, NM * BLK_A + BLK_B, wn * 64 + t * 16);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < IT; ++i) F.a[m][i] = frag(base, m * BLK_A, wm * 16 * IT + i * 16);
  };
  auto mfmas = [&](const Frags& F) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int h = 0; h < NB; ++h)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[m][i][t] = pf_mfma(F.a[m][i], F.b[h][t], acc[m][i][t]);
  };
  // Stage st's fragments are in Fc. Wait for stage st + 1, refill stage st's buffer (every
  // wave has read it) with stage st + NS, read stage st + 1's fragments into Fn, then run Fc
  // on the matrix cores. Past the last stage the refill loads the last stage again (in
  // bounds, never read), so every step has the same loads in flight and no branch.
  auto step = [&](int st, Frags& Fc, Frags& Fn) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * DPS) : "memory");
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);  // this wave's reads of stage st are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(min(st + NS, nk - 1), st % NS);
    read_frags(Fn, st + 1);
    mfmas(Fc);
  };
  static_assert(NS >= 2 && NS <= 4 && (NS - 1) * DPS <= 63, "vmcnt range");
#pragma unroll
  for (int st = 0; st < NS; ++st) issue(min(st, nk - 1), st);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * DPS) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  Frags F0, F1;
  read_frags(F0, 0);
  for (int st = 0; st < nk; st += 2) {  // nk = d / 32 is even
    step(st, F0, F1);
    step(st + 1, F1, F0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in LDS after the loop
  // epilogue: lane holds token 16t + r16 and neurons 16i + 4g .. +3 of the wave's block
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int i0 = m0 + wm * 16 * IT + i * 16 + 4 * g;
    float ba[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ba[j] = (b_act && i0 + j < n) ? b_act[i0 + j] : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = b0 + wn * 64 + t * 16 + r16;
      _Float16 hv[4], lv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float h = acc[0][i][t][j] + ba[j];
        h = h > 0.f ? h : 0.f;
        if (GATED) h *= acc[NM - 1][i][t][j];
        if (i0 + j >= n) h = 0.f;
        hv[j] = (_Float16)h;
        lv[j] = (_Float16)(h - (float)hv[j]);
      }
      const size_t o = (size_t)tok * np + i0;
      *reinterpret_cast<uint2*>(hh + o) = __builtin_bit_cast(uint2, hv);
      if (LO) *reinterpret_cast<uint2*>(hl + o) = __builtin_bit_cast(uint2, lv);
    }
  }
}

// Down projection on the direct-to-LDS pipeline: workgroup (ct, bt, s) computes columns
// [128 ct, +128) x tokens [128 bt, +128) over stages of 32 neurons of its split. Both
// operands go straight from memory to LDS. H rows (tokens, 64 bytes a stage) are swizzled
// as in the up kernel. W_down^T rows (32 neurons x 256 bytes a stage) keep their row-major
// layout with row k's 16-byte chunk c at position c ^ wsw(k); the matrix cores' operand
// (8 consecutive neurons of one column) is read with two LDS transpose reads
// (ds_read_b64_tr_b16): in each 16-lane group, lane i names row k0 + i / 4 at column
// n0 + 4 (i % 4), and lane j receives column n0 + j of rows k0 .. k0 + 3. Wave w takes
// tokens 64 (w & 1) .. +64 and columns 64 (w >> 1) .. +64; two workgroups share a compute
// unit. The loop steps as the up kernel's (the next stage's fragments are read while the
// matrix cores take the current ones); a split with an odd stage count ends on one step.
__device__ __forceinline__ int pf_wsw(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }
template <bool LO>
__global__ __launch_bounds__(TPB) void k_pf_down(const void* __restrict__ w_down_t, int ld_down,
                                               const float* __restrict__ b_out,
                                               const u32x4* __restrict__ hh,
                                               const u32x4* __restrict__ hl, int d, int n,
                                               int np, int B, int Bp, int S,
                                               float* __restrict__ y, float* __restrict__ part) {
  constexpr int NB = LO ? 2 : 1;           // activation halves (hi, lo)
  constexpr int KS = 32;                   // neurons a stage
  constexpr int BLK_W = KS * PF_T;         // halfs: 32 neurons x 128 columns
  constexpr int BLK_H = PF_T * KS;         // halfs: 128 tokens x 32 neurons
  constexpr int STAGE = BLK_W + NB * BLK_H;
  constexpr int NS = LO ? 3 : 4;           // 72 or 64 KB
  constexpr int NGW = BLK_W / 512, NGH = BLK_H / 512;  // 1 KB loads per block
  constexpr int NG = NGW + NB * NGH;
  constexpr int DPS = NG / (TPB / 64);
  static_assert(NG % (TPB / 64) == 0, "whole loads per wave");
  __shared__ __attribute__((aligned(16))) _Float16 sbuf[NS * STAGE];
  const int nct = d / PF_T, nbt = Bp / PF_T;
  const int ct = blockIdx.x % nct, bt = (blockIdx.x / nct) % nbt, s = blockIdx.x / (nct * nbt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int c0 = ct * PF_T, b0 = bt * PF_T;
  const int nks = np / KS;
  const int kb = (int)((long long)nks * s / S), ke = (int)((long long)nks * (s + 1) / S);
  const int nk = ke - kb;
  const u32x4* w = static_cast<const u32x4*>(w_down_t);
  const int hch = np / 8;  // 16-byte chunks of an H row

  const int lr = lane >> 2;                    // H: row within a 16-row group
  const int lc = ((lane & 3) - (lr >> 2)) & 3;  // H: global chunk this lane's position holds
  auto issue = [&](int st, int buf) {
    _Float16* base = sbuf + buf * STAGE;
    const int k0 = (kb + st) * KS;
#pragma unroll
    for (int v = 0; v < DPS; ++v) {
      const int u = wave + (TPB / 64) * v;  // wave-uniform
      const u32x4* src;
      int off;
      if (u < NGW) {
        const int kr = 4 * u + (lane >> 4);
        const int c = (lane & 15) ^ pf_wsw(kr);
        src = w + (size_t)min(k0 + kr, n - 1) * ld_down + c0 / 8 + c;  // neurons past d_ffn meet h = 0
        off = u * 512;
      } else {
        const int o = (u - NGW) / NGH, q = (u - NGW) % NGH;
        src = (o == 0 ? hh : hl) + (size_t)(b0 + q * 16 + lr) * hch + (kb + st) * (KS / 8) + lc;
        off = BLK_W + o * BLK_H + q * 16 * KS;
      }
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(base + off),
                                       16, 0, 0);
    }
  };
  auto hfrag = [&](const _Float16* base, int o, int R) {
    return *reinterpret_cast<const half8_t*>(base + BLK_W + o * BLK_H + R * KS +
                                             (r16 * 4 + ((g + (r16 >> 2)) & 3)) * 8);
  };
  // W operand for columns n0 .. n0 + 15: neurons 8g .. 8g + 7 of column n0 + r16
  auto wfrag = [&](const _Float16* base, int n0) {
    const int col = n0 + 4 * (r16 & 3);
    const int ka = 8 * g + (r16 >> 2), kc = ka + 4;
    const _Float16* pa = base + ka * PF_T + (((col >> 3) ^ pf_wsw(ka)) << 3) + (col & 7);
    const _Float16* pc = base + kc * PF_T + (((col >> 3) ^ pf_wsw(kc)) << 3) + (col & 7);
    const short4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)(pa));
    const short4_t c = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)(pc));
    const half4_t ha = __builtin_bit_cast(half4_t, a), hc = __builtin_bit_cast(half4_t, c);
    return __builtin_shufflevector(ha, hc, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = float4_t{0.f, 0.f, 0.f, 0.f};

  struct Frags {
    half8_t b[4];
    half8_t a[NB][4];
  };
  auto read_frags = [&](Frags& F, int st) {
    const _Float16* base = sbuf + (st % NS) * STAGE;
#pragma unroll
    for (int t = 0; t < 4; ++t) F.b[t] = wfrag(base, wn * 64 + t * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      F.a[0][i] = hfrag(base, 0, wm * 64 + i * 16);
      if constexpr (LO) F.a[NB - 1][i] = hfrag(base, 1, wm * 64 + i * 16);
    }
  };
  auto mfmas = [&](const Frags& F) {
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = pf_mfma(F.a[h][i], F.b[t], acc[i][t]);
  };
  auto step = [&](int st, Frags& Fc, Frags& Fn) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * DPS) : "memory");
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);  // this wave's reads of stage st are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(min(st + NS, nk - 1), st % NS);
    read_frags(Fn, st + 1);
    mfmas(Fc);
  };
  if (nk > 0) {
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(min(st, nk - 1), st);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * DPS) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Frags F0, F1;
    read_frags(F0, 0);
    int st = 0;
    for (; st + 1 < nk; st += 2) {
      step(st, F0, F1);
      step(st + 1, F1, F0);
    }
    if (st < nk) step(st, F0, F1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in LDS after the loop
  }
  // lane holds column 16t + r16 and tokens 16i + 4g .. +3 of the wave's block
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int col = c0 + wn * 64 + t * 16 + r16;
    const float bo = (S == 1 && b_out) ? b_out[col] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = b0 + wm * 64 + i * 16 + 4 * g + j;
        if (S == 1) {
          if (tok < B) y[(size_t)tok * d + col] = acc[i][t][j] + bo;
        } else {
          part[((size_t)s * Bp + tok) * d + col] = acc[i][t][j];
        }
      }
  }
}

// y[b][c] = sum over s in order of part[s][b][c], + b_out[c], for the chunk's B tokens
__global__ __launch_bounds__(TPB) void k_pf_sum(const float* __restrict__ part, int S, int B,
                                                int Bp, int d, const float* __restrict__ b_out,
                                                float* __restrict__ y) {
  const size_t total = (size_t)B * d;
  for (size_t q = (size_t)blockIdx.x * TPB + threadIdx.x; q < total; q += (size_t)gridDim.x * TPB) {
    float a = part[q];
    for (int s = 1; s < S; ++s) a += part[(size_t)s * Bp * d + q];
    y[q] = a + (b_out ? b_out[q % d] : 0.f);
  }
}

template <bool GATED, int IT, bool LO>
void pf_up_launch(const LayerDev& L, const u32x4* xh, const u32x4* xl, int np, int nbt,
                  _Float16* hh, _Float16* hl, hipStream_t s) {
  const int nmt = np / (32 * IT);
  hipLaunchKernelGGL((k_pf_up<GATED, IT, LO>), dim3((nmt + 7) / 8 * 8 * nbt), dim3(TPB), 0, s,
                     L.w_act, L.act_ld, L.b_act, xh, xl, L.d, L.n, np, nmt, hh, hl);
}

template <bool LO>
void pf_chunk(const LayerDev& L, const float* xc, int bc, int Bp, float* yc, u32x4* xh,
              u32x4* xl, _Float16* hh, _Float16* hl, float* part, hipStream_t s) {
  const int d = L.d, n = L.n;
  const int nct = d / PF_T;
  const int items = Bp * (d / 8);
  hipLaunchKernelGGL(k_pf_split<LO>, dim3(std::min((items + TPB - 1) / TPB, 4 * L.n_cus)),
                     dim3(TPB), 0, s, xc, bc, Bp, d, xh, xl);
  const int nbt = Bp / PF_T;
  // up tile and down splits: the plan of sffn_host.h (pf_up_it, pf_splits)
  const int it = host::pf_up_it(n, L.gated, LO, nbt, L.n_cus);
  const int np = host::pf_np(n, it);  // H row length: whole neuron tiles
  if (L.gated) {
    if (it == 3) pf_up_launch<true, 3, LO>(L, xh, xl, np, nbt, hh, hl, s);
    else pf_up_launch<true, 2, LO>(L, xh, xl, np, nbt, hh, hl, s);
  } else {
    if (it == 6) pf_up_launch<false, 6, LO>(L, xh, xl, np, nbt, hh, hl, s);
    else if (it == 4) pf_up_launch<false, 4, LO>(L, xh, xl, np, nbt, hh, hl, s);
    else pf_up_launch<false, 2, LO>(L, xh, xl, np, nbt, hh, hl, s);
  }
  const int S = host::pf_splits(d, L.n_cus, nbt, (size_t)np);
  hipLaunchKernelGGL(k_pf_down<LO>, dim3(nct * nbt * S), dim3(TPB), 0, s, L.w_down_t, L.down_ld,
                     L.b_out, reinterpret_cast<const u32x4*>(hh), reinterpret_cast<const u32x4*>(hl),
                     d, n, np, bc, Bp, S, yc, part);
  if (S > 1) {
    const size_t tot = (size_t)bc * d;
    hipLaunchKernelGGL(k_pf_sum, dim3((unsigned)std::min<size_t>((tot + TPB - 1) / TPB, 8 * L.n_cus)),
                       dim3(TPB), 0, s, part, S, bc, Bp, d, L.b_out, yc);
  }
}

}  // namespace

bool prefill_ok(const LayerDev& L) { return L.w_f16 && L.d % PF_T == 0 && L.d <= 65536; }

// scratch for chunks of up to `chunk` tokens (rounded up to 128)
size_t prefill_work_bytes(const LayerDev& L, int chunk) {
  return host::pf_work_bytes(L.d, L.n, L.n_cus, chunk);
}

// tokens the scratch holds per chunk (a multiple of 128; 0 when not even 128)
int prefill_chunk(const LayerDev& L, size_t work_bytes) {
  return host::pf_chunk_tokens(L.d, L.n, L.n_cus, work_bytes);
}

hipError_t run_prefill(const LayerDev& L, const float* x, int B, float* y, void* work,
                       size_t work_bytes, bool fp16_act, hipStream_t s) {
  const int chunk = prefill_chunk(L, work_bytes);
  if (chunk < PF_T) return hipErrorInvalidValue;
  const int d = L.d, n = L.n;
  for (int b0 = 0; b0 < B; b0 += chunk) {
    const int bc = std::min(chunk, B - b0);
    const int Bp = (bc + PF_T - 1) / PF_T * PF_T;
    char* p = static_cast<char*>(work);
    const host::PfCarve c = host::pf_carve(d, n, L.n_cus, (size_t)Bp);  // within work_bytes
    u32x4* xh = reinterpret_cast<u32x4*>(p + c.xh);
    u32x4* xl = reinterpret_cast<u32x4*>(p + c.xl);
    _Float16* hh = reinterpret_cast<_Float16*>(p + c.hh);  // rows np <= pf_rows(n)
    _Float16* hl = reinterpret_cast<_Float16*>(p + c.hl);
    float* part = reinterpret_cast<float*>(p + c.part);
    const float* xc = x + (size_t)b0 * d;
    float* yc = y + (size_t)b0 * d;
    if (fp16_act)
      pf_chunk<false>(L, xc, bc, Bp, yc, xh, xl, hh, hl, part, s);
    else
      pf_chunk<true>(L, xc, bc, Bp, yc, xh, xl, hh, hl, part, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sffn
