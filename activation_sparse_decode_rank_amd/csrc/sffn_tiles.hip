// Predictor scores, threshold and compaction as separate kernels (the standalone entry
// points and the batch path), and the gathered-tile up and down projections on the matrix
// cores for batches of 2 or more tokens with fp16 weights and d a multiple of 256 (gfx950).
#include "sffn_device.h"

namespace sffn {
namespace {

// scores[b][i] = P2[i] . q_b + c_i for rows [row_begin, row_end) of this workgroup.
template <bool PF16, int L, int CPLP, int PASSES>
__global__ __launch_bounds__(TPB) void k_pred_scores(const void* __restrict__ p2,
                                                     const float* __restrict__ pbias,
                                                     const float* __restrict__ q, int n, int r,
                                                     int B, float* __restrict__ scores) {
  constexpr int EPC = Elt<PF16>::EPC;
  constexpr int RPP = TPB / L;
  const int tid = threadIdx.x;
  const int g = tid / L, gl = tid % L;
  const int nchp = r / EPC;
  const int row_base = blockIdx.x * RPP * PASSES;
  u32x4 wv[PASSES][CPLP];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = row_base + p * RPP + g;
#pragma unroll
    for (int m = 0; m < CPLP; ++m) {
      const int c = gl + m * L;
      if (row < n && c < nchp) wv[p][m] = ld_chunk(p2, (size_t)row * nchp + c);
    }
  }
  for (int b = 0; b < B; ++b) {
    float qs[CPLP][EPC];
#pragma unroll
    for (int m = 0; m < CPLP; ++m) {
      const int c = gl + m * L;
      if (c < nchp) load_x<EPC>(q + (size_t)b * r + (size_t)c * EPC, qs[m]);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = row_base + p * RPP + g;
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < CPLP; ++m) {
        const int c = gl + m * L;
        if (c < nchp && row < n) acc = dot_chunk<PF16>(wv[p][m], qs[m], acc);
      }
      acc = group_sum<L>(acc);
      if (gl == group_leader(L) && row < n) scores[(size_t)b * n + row] = acc + (pbias ? pbias[row] : 0.f);
    }
  }
}

// ============================================================================ compaction
// Pass 1, one thread per neuron: token bits and the union ballot word of every 64 neurons.
__global__ __launch_bounds__(TPB) void k_cmp_tiles(const float* __restrict__ scores, int n,
                                                   int B, float tau,
                                                   uint64_t* __restrict__ tok_full,
                                                   uint64_t* __restrict__ words) {
  const int i = blockIdx.x * TPB + threadIdx.x;
  const int lane = threadIdx.x & 63;
  uint64_t bits = 0;
  if (i < n)
    for (int b = 0; b < B; ++b)
      if (scores[(size_t)b * n + i] > tau) bits |= (uint64_t)1 << b;  // NaN compares false
  const uint64_t word = __ballot(bits != 0);
  if (i < n) {
    tok_full[i] = bits;
    if (lane == 0) words[i >> 6] = word;
  }
}

// Pass 2, 256-neuron tiles: the exclusive prefix of the union words' popcounts before the
// tile, then every active neuron writes itself at its ascending position. The last tile
// writes the total.
__global__ __launch_bounds__(TPB) void k_cmp_scatter(const uint64_t* __restrict__ tok_full,
                                                     const uint64_t* __restrict__ words, int n,
                                                     int n_tiles, int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ count,
                                                     uint64_t* __restrict__ tokmask) {
  __shared__ int s_off;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = (n + 63) / 64;
  if (threadIdx.x < 64) {
    int acc = 0;
    for (int u = lane; u < 4 * t; u += 64) acc += __popcll(words[u]);
    acc = wave_incl_scan(acc);
    if (lane == 63) s_off = acc;
  }
  __syncthreads();
  const int i = t * TPB + threadIdx.x;
  if (i < n) {
    const uint64_t word = words[i >> 6];
    if ((word >> lane) & 1) {
      int before = 0;
      for (int v = 0; v < wave; ++v) before += __popcll(words[t * 4 + v]);
      const uint64_t lower = lane ? (word & ((~(uint64_t)0) >> (64 - lane))) : 0;
      const int k = s_off + before + __popcll(lower);
      idx[k] = i;
      if (tokmask) tokmask[k] = tok_full[i];
    }
  }
  if (t == n_tiles - 1 && threadIdx.x == 0) {
    int tot = s_off;
    for (int v = 0; v < 4; ++v)
      if (4 * t + v < nw) tot += __popcll(words[4 * t + v]);
    *count = tot;
  }
}

// Predictor stage 2, threshold and the union words at batch, on the matrix cores (the
// first compaction pass fused in). Workgroup w owns neurons [64w, 64w + 64), wave v the 16
// from 64w + 16v. With v_mfma_f32_16x16x4_f32 (lane l: A[l%16][l/16], B[l/16][l%16];
// result column l%16, rows 4*(l/16)..+3), lane group g = l/16 takes the 16-byte P2 chunks
// 4u + g (u = 0, 1, ...) of its row, so each load instruction reads 64 contiguous bytes of
// each of the wave's 16 rows, and each product takes one k from each group. q sits in LDS
// k-major, token pitch TP = 16 NT rounded up to 32, token b of row k at column
// b ^ (16 * (chunk of k & 1)): a wave's 64 reads of one step then fall two to a bank.
// Products and sums are fp32. A ballot of every thresholded result register gives 16
// tokens x 4 neurons of bits at once. Writes tok_full and the union word (as k_cmp_tiles
// does) and, if asked, the scores.
template <bool PF16, int NT>
__global__ __launch_bounds__(TPB) void k_score_tiles(const void* __restrict__ p2,
                                                     const float* __restrict__ pbias,
                                                     const float* __restrict__ q, int n, int r,
                                                     int B, float tau,
                                                     uint64_t* __restrict__ tok_full,
                                                     uint64_t* __restrict__ words,
                                                     float* __restrict__ scores) {
  constexpr int EPC = Elt<PF16>::EPC;
  constexpr int CU = 8;  // P2 chunks per lane in flight
  constexpr int TP = (16 * NT + 31) / 32 * 32;  // a multiple of 32, so b ^ 16 stays in the row
  extern __shared__ float s_q[];  // [r][TP]
  __shared__ uint64_t s_tok[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int kg = r / 4;           // k values per lane group
  const int base = blockIdx.x * 64 + wave * 16;
  const int row = min(base + r16, n - 1);
  const int nck = kg / EPC;       // P2 chunks per lane
  const size_t c0 = (size_t)row * (r / EPC) + g;   // chunk 4u + g of the row
  // q comes from the previous kernel through the last-level cache. Its first batch of QB
  // items per thread (item (k4, b) = 4 consecutive k of token b, clamped to B - 1) and the
  // first batch of P2 loads all go out before anything waits; then q is stored to LDS
  constexpr int QB = 8;
  const int nq = (r / 4) * TP;
  float4_t qv[QB];
  auto q_load = [&](int u0) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int u = min(u0 + j * TPB + tid, nq - 1);
      const int b = u % TP, k4 = u / TP;
      qv[j] = *reinterpret_cast<const float4_t*>(q + (size_t)min(b, B - 1) * r + 4 * k4);
    }
  };
  // items past the end repeat the last item (same value to the same place), so the
  // stores carry no branch that the compiler could sink a load into
  auto q_store = [&](int u0) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int u = min(u0 + j * TPB + tid, nq - 1);
      const int b = u % TP, k4 = u / TP;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * k4 + e;
        s_q[k * TP + (b ^ (16 * ((k / EPC) & 1)))] = qv[j][e];
      }
    }
  };
  q_load(0);
  u32x4 wv[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) wv[u] = ld_stream(p2, c0 + 4 * (size_t)min(u, nck - 1));
  __builtin_amdgcn_sched_barrier(0);
  q_store(0);
  for (int u0 = QB * TPB; u0 < nq; u0 += QB * TPB) {
    q_load(u0);
    q_store(u0);
  }
  const float* qb[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) qb[tt] = s_q + (size_t)g * EPC * TP + ((16 * tt + r16) ^ (16 * (g & 1)));
  __syncthreads();
  float4_t acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int cb = 0; cb < nck; cb += CU) {
    if (cb > 0) {
#pragma unroll
      for (int u = 0; u < CU; ++u) wv[u] = ld_stream(p2, c0 + 4 * (size_t)min(cb + u, nck - 1));
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      if (cb + u < nck) {  // uniform
        float f[EPC];
        unpack<PF16>(wv[u], f);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const float* qp = qb[tt] + (size_t)(cb + u) * 4 * EPC * TP;
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(f[e], qp[e * TP], acc[tt], 0, 0, 0);
        }
      }
    }
  }
  // scores and threshold: lane holds tokens 16tt + l%16, neurons base + 4g + v
  float pb[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int i = base + 4 * g + v;
    pb[v] = (pbias && i < n) ? pbias[i] : 0.f;
  }
  uint64_t bits = 0;  // lanes 0..15: token bits of neuron base + lane
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int b = 16 * tt + r16;
    uint64_t m[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = base + 4 * g + v;
      const float sc = acc[tt][v] + pb[v];
      if (scores && b < B && i < n) scores[(size_t)b * n + i] = sc;
      m[v] = __ballot(b < B && i < n && sc > tau);  // NaN compares false
    }
    // neuron base + lane (lane < 16) = 4G + v with G = lane / 4: its 16 token bits sit at
    // bits 16G .. 16G + 15 of ballot v
    const int v = lane & 3, G = (lane >> 2) & 3;
    const uint64_t mv = v == 0 ? m[0] : v == 1 ? m[1] : v == 2 ? m[2] : m[3];
    bits |= ((mv >> (16 * G)) & 0xFFFFull) << (16 * tt);
  }
  if (lane < 16) s_tok[wave * 16 + lane] = bits;
  __syncthreads();
  if (wave == 0) {
    const int i = blockIdx.x * 64 + lane;
    const uint64_t tb = i < n ? s_tok[lane] : 0;
    const uint64_t word = __ballot(tb != 0);
    if (i < n) tok_full[i] = tb;
    if (lane == 0) words[blockIdx.x] = word;
  }
}

// ============================================================================ batch tiles
// From TILE_MIN_B tokens on, the union rows form dense tiles and the products go to the
// matrix cores: v_mfma_f32_16x16x32_f16 multiplies a 16x32 fp16 tile by a 32x16 fp16 tile
// into 16x16 fp32 accumulators (lane l holds row l%16, k 8*(l/16)..+7 of the left operand,
// column l%16 and the same k of the right one; the result lands as column l%16, rows
// 4*(l/16)..+3). Weights are fp16 as stored; fp32 activations enter as a hi + lo pair of
// fp16 values (v = hi + lo to about 22 significant bits), two products per tile.

__device__ __forceinline__ float4_t mfma16(const half8_t& a, const half8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Up projection over the union list. Workgroup iteration u takes the TR tiles of 16 listed
// neurons from u*TR on, for all B tokens: wave w of its W sums input columns
// [w*d/W, (w+1)*d/W) for all TR tiles (each activation fragment serves TR tiles), the W
// partial tiles are added in wave order through LDS, then wave i < TR applies bias, ReLU
// (gated: times the up tile) and the token bits to tile i and writes hT[b*ldh + p]
// (token-major, for the down projection's left operand).
// Weights are read whole lines at a time (lane l: row l/8 of an 8-row half tile, 16-byte
// chunk l%8 of each 128-byte piece): the operand layout itself (lane l: row l%16, chunk
// l/16) would read 16 rows x 64 bytes per instruction, which streams gathered rows at about
// two thirds of the rate. Each 64-input step pair passes through a small wave-private LDS
// buffer into operand order. The activations come split in x_hl (the token fastest), so a
// wave's operand load for one k-step is one contiguous run of B x 64 bytes. Loads run one batch of KP
// step pairs ahead of the products.
constexpr int FW_WORDS_MAX = 1024;  // union words the up kernel can list itself (n <= 65536)

// The list from the union words (FW): each workgroup prefix-sums the popcounts of the
// words in LDS, and list position p is the k-th set bit of the word w with
// pref[w] <= p < pref[w + 1] (found by binary search over the prefixes; empty words share
// their successor's prefix and are never chosen). The positions of its own tiles are
// written to idx, with their token bits; workgroup 0 writes the count.
template <bool GATED, int NT, int TR, int W, bool FW, bool HALF>
__global__ __launch_bounds__(64 * W) void k_up_mfma(const void* __restrict__ w_act, int ld_act,
                                                    const float* __restrict__ b_act,
                                                    const u32x4* __restrict__ x_hl, int d,
                                                    int n, int B, int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ count,
                                                    uint64_t* __restrict__ tokmask,
                                                    const uint64_t* __restrict__ words,
                                                    const uint64_t* __restrict__ tok_full,
                                                    float* __restrict__ hT, int ldh,
                                                    float* __restrict__ y0, int ny) {
  constexpr int NM = GATED ? 2 : 1;
  constexpr int KP = (NT == 1 && TR == 1) ? 2 : 1;    // 64-input step pairs per load batch
  constexpr int PITCH = 9;                            // transpose buffer row pitch in chunks
  // rows per workgroup iteration; HALF: 8 listed rows a tile (rows 8..15 of each operand
  // tile stay zero and their results are dropped), so a small union spreads over twice the
  // workgroups
  constexpr int RT = HALF ? 8 : 16 * TR;
  static_assert(!HALF || TR == 1, "half tiles take one row tile");
  __shared__ u32x4 s_w[W][KP][TR][NM][16 * PITCH];
  __shared__ float4_t s_acc[W][TR][NM][NT][64];
  for (int i = blockIdx.x * 64 * W + threadIdx.x; i < ny; i += gridDim.x * 64 * W) y0[i] = 0.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;
  constexpr int NTH = 64 * W;
  constexpr int PE = FW ? (FW_WORDS_MAX + NTH - 1) / NTH : 1;  // words per thread in the scan
  __shared__ int32_t s_pref[FW ? FW_WORDS_MAX + 1 : 1];
  __shared__ uint64_t s_word[FW ? FW_WORDS_MAX : 1];
  __shared__ int32_t s_rows[FW ? RT : 1];
  __shared__ int32_t s_wsum[W];
  const int nw = (n + 63) / 64;
  int ia[TR], ib[TR];
  int cnt;
  if constexpr (FW) {
    // thread t loads words t*PE .. t*PE + PE - 1 together (one round trip, any n)
    int loc[PE], sum = 0;
#pragma unroll
    for (int e = 0; e < PE; ++e) {
      const int w = tid * PE + e;
      const uint64_t v = words[min(w, nw - 1)];
      s_word[w] = v;
      loc[e] = w < nw ? __popcll(v) : 0;
      sum += loc[e];
    }
    const int incl = wave_incl_scan(sum);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int run = incl - sum, total = 0;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      run += v < wave ? s_wsum[v] : 0;
      total += s_wsum[v];
    }
#pragma unroll
    for (int e = 0; e < PE; ++e) {
      const int w = tid * PE + e;
      if (w < nw) s_pref[w] = run;
      run += loc[e];
    }
    if (tid == 0) s_pref[nw] = total;
    if (blockIdx.x == 0 && tid == 0) *count = total;
    cnt = min(total, n);
    __syncthreads();
  } else {
    // the count and the first iteration's list entries load together: entries past the
    // count are stale but clamped to a valid row below, and their results are never stored
    const int cnt_raw = *count;
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      ia[i] = idx[min((int)blockIdx.x * RT + 16 * i + lr, n - 1)];
      ib[i] = HALF ? 0 : idx[min((int)blockIdx.x * RT + 16 * i + 8 + lr, n - 1)];
    }
    cnt = min(max(cnt_raw, 0), n);
  }
  const int nch = d / 8;                 // chunks per matrix row
  const int qch = nch / W;               // this wave's chunks of each row
  const int npairs = qch / 8;            // its 64-input step pairs
  const int c0 = wave * qch;
  const u32x4* wbase = reinterpret_cast<const u32x4*>(w_act);
  // x_hl holds exactly B token slots per chunk; lanes of token tile columns past the batch
  // re-read the last token's chunk (their products are never stored), so at a few tokens
  // an operand load touches one or two cache lines, not a padded kilobyte
  const u32x4* xh = x_hl;
  const u32x4* xl = x_hl + (size_t)nch * B;
  int tok[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) tok[tt] = min(16 * tt + r16, B - 1);
  u32x4* sw = &s_w[wave][0][0][0][0];
  if constexpr (HALF) {
    // rows 8..15 of every operand tile buffer: zero once, never written again
    for (int q = lane; q < KP * TR * NM * 8 * PITCH; q += 64)
      sw[(q / (8 * PITCH)) * 16 * PITCH + 8 * PITCH + q % (8 * PITCH)] = u32x4{0u, 0u, 0u, 0u};
  }
  const int et = wave < TR ? wave : 0;   // the tile whose epilogue this wave finishes
  for (int u = blockIdx.x; u * RT < cnt; u += gridDim.x) {
    if constexpr (FW) {
      if (tid < RT) {
        const int p = min(u * RT + tid, cnt - 1);
        int lo = 0, hi = nw - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pref[mid] <= p) lo = mid;
          else hi = mid - 1;
        }
        uint64_t v = s_word[lo];
        int k = p - s_pref[lo], bit = 0;
#pragma unroll
        for (int sft = 32; sft >= 1; sft >>= 1) {
          const uint64_t low = (((uint64_t)1) << sft) - 1;
          const int c = __popcll(v & low);
          if (k >= c) {
            k -= c;
            v >>= sft;
            bit += sft;
          } else {
            v &= low;
          }
        }
        const int row = lo * 64 + bit;
        s_rows[tid] = row;
        if (u * RT + tid < cnt) {
          idx[u * RT + tid] = row;
          if (tokmask) tokmask[u * RT + tid] = tok_full[row];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TR; ++i) {
        ia[i] = s_rows[16 * i + lr];
        ib[i] = HALF ? 0 : s_rows[16 * i + 8 + lr];
      }
    } else if (u != (int)blockIdx.x) {
#pragma unroll
      for (int i = 0; i < TR; ++i) {
        ia[i] = idx[min(u * RT + 16 * i + lr, cnt - 1)];
        ib[i] = HALF ? 0 : idx[min(u * RT + 16 * i + 8 + lr, cnt - 1)];
      }
    }
    const u32x4* pa[TR];
    const u32x4* pb[TR];
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      pa[i] = wbase + (size_t)((ia[i] >= 0 && ia[i] < n) ? ia[i] : 0) * ld_act + c0 + lc;
      pb[i] = wbase + (size_t)((ib[i] >= 0 && ib[i] < n) ? ib[i] : 0) * ld_act + c0 + lc;
    }
    float4_t acc[TR][NM][NT];
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[i][m][tt] = float4_t{0.f, 0.f, 0.f, 0.f};
    u32x4 wa[2][KP][TR][NM], wb[2][KP][TR][NM], xv[2][KP][2][NT][2];
    // KP pairs into buffer bb; every load unconditional (pair index clamped)
    auto load = [&](int p0, int bb) {
#pragma unroll
      for (int kp = 0; kp < KP; ++kp) {
        const int p = min(p0 + kp, npairs - 1);
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            wa[bb][kp][i][m] = ld_stream(pa[i], (size_t)m * nch + 8 * p);
            if constexpr (!HALF) wb[bb][kp][i][m] = ld_stream(pb[i], (size_t)m * nch + 8 * p);
          }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const size_t c = (size_t)(c0 + 8 * p + 4 * st + g) * B;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            xv[bb][kp][st][tt][0] = xh[c + tok[tt]];
            xv[bb][kp][st][tt][1] = xl[c + tok[tt]];
          }
        }
      }
    };
    // products of the first KPN pairs held in buffer bb (all of them live: no selects)
    auto mult = [&](int bb, auto kpn) {
      constexpr int KPN = decltype(kpn)::value;
#pragma unroll
      for (int kp = 0; kp < KPN; ++kp)
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            u32x4* bw = sw + ((kp * TR + i) * NM + m) * 16 * PITCH;
            bw[lr * PITCH + lc] = wa[bb][kp][i][m];
            if constexpr (!HALF) bw[(8 + lr) * PITCH + lc] = wb[bb][kp][i][m];
          }
      wave_lds_sync();
#pragma unroll
      for (int kp = 0; kp < KPN; ++kp)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < TR; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              const half8_t w8 = __builtin_bit_cast(
                  half8_t, sw[((kp * TR + i) * NM + m) * 16 * PITCH + r16 * PITCH + 4 * st + g]);
#pragma unroll
              for (int tt = 0; tt < NT; ++tt) {
                acc[i][m][tt] = mfma16(w8, __builtin_bit_cast(half8_t, xv[bb][kp][st][tt][0]), acc[i][m][tt]);
                acc[i][m][tt] = mfma16(w8, __builtin_bit_cast(half8_t, xv[bb][kp][st][tt][1]), acc[i][m][tt]);
              }
            }
      wave_lds_sync();
    };
    // whole iterations of 2 KP pairs, pipelined (the scheduling barriers keep each batch's
    // loads ahead of the products before their use; the scheduler would otherwise sink
    // them to their first use), the last one peeled; then the leftover pairs one at a time
    const int nfull = npairs / (2 * KP) * (2 * KP);
    // the epilogue's list entries, token bits and biases (lane: positions 4g + j of tile
    // et) go out behind the first weight batch; by the time they are used they have long
    // landed
    int ej[4];
    uint64_t em[4];
    float eb[4];
    auto load_epilogue = [&]() {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (FW) {
          ej[j] = s_rows[min(16 * et + 4 * g + j, RT - 1)];
          em[j] = tok_full[ej[j]];
        } else {
          const int pc = min(u * RT + 16 * et + 4 * g + j, cnt - 1);
          ej[j] = idx[pc];
          // token bits by list position; else by neuron from the compaction (decode with no
          // caller mask); else every token uses every listed neuron (standalone forward)
          em[j] = tokmask ? tokmask[pc]
                          : tok_full ? tok_full[(ej[j] >= 0 && ej[j] < n) ? ej[j] : 0]
                                     : ~(uint64_t)0;
        }
        eb[j] = (b_act && ej[j] >= 0 && ej[j] < n) ? b_act[ej[j]] : 0.f;
      }
    };
    if (nfull > 0) {
      load(0, 0);
      load_epilogue();
      int p0 = 0;
      for (; p0 + 2 * KP < nfull; p0 += 2 * KP) {
        load(p0 + KP, 1);
        __builtin_amdgcn_sched_barrier(0);
        mult(0, std::integral_constant<int, KP>{});
        __builtin_amdgcn_sched_barrier(0);
        load(p0 + 2 * KP, 0);
        __builtin_amdgcn_sched_barrier(0);
        mult(1, std::integral_constant<int, KP>{});
        __builtin_amdgcn_sched_barrier(0);
      }
      // the last whole iteration fetches nothing ahead (a wave retires only when its loads
      // have landed)
      load(p0 + KP, 1);
      __builtin_amdgcn_sched_barrier(0);
      mult(0, std::integral_constant<int, KP>{});
      __builtin_amdgcn_sched_barrier(0);
      mult(1, std::integral_constant<int, KP>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nfull == 0) load_epilogue();
    for (int p = nfull; p < npairs; ++p) {
      load(p, 0);
      mult(0, std::integral_constant<int, 1>{});
    }
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) s_acc[wave][i][m][tt][lane] = acc[i][m][tt];
    __syncthreads();
    if (wave < TR) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        float4_t v[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          v[m] = s_acc[0][et][m][tt][lane];
#pragma unroll
          for (int ww = 1; ww < W; ++ww) v[m] += s_acc[ww][et][m][tt][lane];
        }
        const int b = tt * 16 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = u * RT + 16 * et + 4 * g + j;
          if (p < cnt && b < B && (!HALF || g < 2)) {
            const bool ok = ej[j] >= 0 && ej[j] < n;
            const float a0 = v[0][j] + eb[j];
            float h = a0 > 0.f ? a0 : 0.f;
            if (GATED) h *= v[NM - 1][j];
            const bool on = (em[j] >> b) & 1;
            hT[(size_t)b * ldh + p] = (ok && on) ? h : 0.f;
          }
        }
      }
    }
    __syncthreads();
  }
}

// Stream-K form of the up projection in the decode step (union listed from the words).
// The work is the list's tiles of TR 16-row tiles times their KBT input blocks (block kb
// of a tile: wave w sums its pairs 2 (kb W + w) and 2 (kb W + w) + 1 of 64 inputs each,
// each activation fragment serving the TR row tiles), flattened tile-major. Workgroup g of the G' = min(G, 2 x tiles) that take
// part gets the equal contiguous range [g T / G', (g + 1) T / G') of the T blocks, so every
// compute unit streams about the same bytes whatever the union's size: whole tiles per
// workgroup leave compute units idle when there are fewer tiles than workgroups, and give
// a few a second round when there are slightly more. Loads run one pair ahead across
// block and tile boundaries.
// A range is at least half a tile long, so a tile has at most 3 parts. A tile inside one
// range is finished there. A part of a split tile (at most two per workgroup: the tile
// its range starts in and the one it ends in) has its W-wave sum published with
// device-coherent stores in slot 2g (the range's first tile) or 2g + 1 (its last), one
// sub-slot per row tile; the part that arrives last at the row tile's counter (wave i
// finishes row tile i) adds the parts in workgroup order (the sum
// does not depend on arrival order), finishes the epilogue, writes the tile's list
// entries and resets the counter to zero for the next call.
constexpr int SK_TMAX = 16;   // tiles one range may touch (listed in LDS at once)
constexpr int SK_PMAX = 3;    // parts of one tile
template <bool GATED, int NT, int TR, int W>
__global__ __launch_bounds__(64 * W) void k_up_sk(const void* __restrict__ w_act, int ld_act,
                                                  const float* __restrict__ b_act,
                                                  const u32x4* __restrict__ x_hl, int d,
                                                  int n, int B, int32_t* __restrict__ idx,
                                                  int32_t* __restrict__ count,
                                                  uint64_t* __restrict__ tokmask,
                                                  const uint64_t* __restrict__ words,
                                                  const uint64_t* __restrict__ tok_full,
                                                  float* __restrict__ hT, int ldh,
                                                  float* __restrict__ y0, int ny,
                                                  float* __restrict__ part,
                                                  int32_t* __restrict__ tcnt) {
  constexpr int NM = GATED ? 2 : 1;
  constexpr int PITCH = 9;
  constexpr int NTH = 64 * W;
  constexpr int PE = (FW_WORDS_MAX + NTH - 1) / NTH;
  constexpr int RT = 16 * TR;            // rows per tile (TR row tiles of 16)
  constexpr int NO = NM * NT * 4 * 64;   // floats of one part of one row tile
  static_assert(SK_TMAX * RT <= NTH, "one listing pass");
  __shared__ u32x4 s_w[W][TR][NM][16 * PITCH];
  __shared__ float4_t s_acc[W][TR][NM][NT][64];
  __shared__ int32_t s_pref[FW_WORDS_MAX + 1];
  __shared__ uint64_t s_word[FW_WORDS_MAX];
  __shared__ int32_t s_rows[SK_TMAX * RT];
  __shared__ int32_t s_wsum[W];
  for (int i = blockIdx.x * NTH + threadIdx.x; i < ny; i += gridDim.x * NTH) y0[i] = 0.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;
  const int nw = (n + 63) / 64;
  // ---- prefix sums of the union words (each thread loads its PE words in one batch)
  int loc[PE], sum = 0;
#pragma unroll
  for (int e = 0; e < PE; ++e) {
    const int w = tid * PE + e;
    const uint64_t v = words[min(w, nw - 1)];
    s_word[w] = v;
    loc[e] = w < nw ? __popcll(v) : 0;
    sum += loc[e];
  }
  const int incl = wave_incl_scan(sum);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
#pragma unroll
  for (int v = 0; v < W; ++v) {
    run += v < wave ? s_wsum[v] : 0;
    total += s_wsum[v];
  }
#pragma unroll
  for (int e = 0; e < PE; ++e) {
    const int w = tid * PE + e;
    if (w < nw) s_pref[w] = run;
    run += loc[e];
  }
  if (tid == 0) s_pref[nw] = total;
  if (blockIdx.x == 0 && tid == 0) *count = total;
  const int cnt = min(total, n);
  __syncthreads();
  // ---- this workgroup's range of blocks
  const int nch = d / 8;
  const int KBT = nch / (16 * W);
  const int ntiles = (cnt + RT - 1) / RT;
  const long long T = (long long)ntiles * KBT;
  const int G = min((int)gridDim.x, 2 * ntiles);
  const int gi = blockIdx.x;
  if (gi >= G) return;  // uniform; also covers an empty list
  auto start_of = [&](long long gg) { return gg * T / G; };
  auto owner_of = [&](long long j) { return (int)(((j + 1) * G - 1) / T); };
  const long long j0 = start_of(gi), j1 = start_of(gi + 1);
  const int t_first = (int)(j0 / KBT), t_last = (int)((j1 - 1) / KBT);
  // ---- rows of tiles t_first .. t_last: list position p is the k-th set bit of the word
  // w with pref[w] <= p < pref[w + 1] (binary search over the prefixes)
  if (tid < (t_last - t_first + 1) * RT) {
    const int p = min(t_first * RT + tid, cnt - 1);
    int lo = 0, hi = nw - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    uint64_t v = s_word[lo];
    int k = p - s_pref[lo], bit = 0;
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) {
      const uint64_t low = (((uint64_t)1) << sft) - 1;
      const int c = __popcll(v & low);
      if (k >= c) {
        k -= c;
        v >>= sft;
        bit += sft;
      } else {
        v &= low;
      }
    }
    s_rows[tid] = lo * 64 + bit;
  }
  __syncthreads();
  // ---- the stream
  const u32x4* wbase = reinterpret_cast<const u32x4*>(w_act);
  const u32x4* xh = x_hl;
  const u32x4* xl = x_hl + (size_t)nch * B;
  int tok[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) tok[tt] = min(16 * tt + r16, B - 1);
  u32x4* sw = &s_w[wave][0][0][0];
  const u32x4* pa[TR];
  const u32x4* pb[TR];
  auto set_rows = [&](int t) {
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      const int ra = s_rows[(t - t_first) * RT + 16 * i + lr];
      const int rb = s_rows[(t - t_first) * RT + 16 * i + 8 + lr];
      pa[i] = wbase + (size_t)((ra >= 0 && ra < n) ? ra : 0) * ld_act + lc;
      pb[i] = wbase + (size_t)((rb >= 0 && rb < n) ? rb : 0) * ld_act + lc;
    }
  };
  u32x4 wa[2][TR][NM], wb[2][TR][NM], xv[2][2][NT][2];
  // pair q (of the row's d / 64) of the current rows into buffer bb
  auto load = [&](int q, int bb) {
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        wa[bb][i][m] = ld_stream(pa[i], (size_t)m * nch + 8 * q);
        wb[bb][i][m] = ld_stream(pb[i], (size_t)m * nch + 8 * q);
      }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const size_t c = (size_t)(8 * q + 4 * st + g) * B;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        xv[bb][st][tt][0] = xh[c + tok[tt]];
        xv[bb][st][tt][1] = xl[c + tok[tt]];
      }
    }
  };
  float4_t acc[TR][NM][NT];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[i][m][tt] = float4_t{0.f, 0.f, 0.f, 0.f};
  auto mult = [&](int bb) {
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        u32x4* bw = sw + (i * NM + m) * 16 * PITCH;
        bw[lr * PITCH + lc] = wa[bb][i][m];
        bw[(8 + lr) * PITCH + lc] = wb[bb][i][m];
      }
    wave_lds_sync();
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < TR; ++i)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const half8_t w8 = __builtin_bit_cast(
              half8_t, sw[(i * NM + m) * 16 * PITCH + r16 * PITCH + 4 * st + g]);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            acc[i][m][tt] = mfma16(w8, __builtin_bit_cast(half8_t, xv[bb][st][tt][0]), acc[i][m][tt]);
            acc[i][m][tt] = mfma16(w8, __builtin_bit_cast(half8_t, xv[bb][st][tt][1]), acc[i][m][tt]);
          }
        }
    wave_lds_sync();
  };
  // epilogue inputs of row tile et of tile t (positions 4g + j): rows, token bits, biases;
  // wave et < TR finishes row tile et
  const int et = wave < TR ? wave : 0;
  int ej[4];
  uint64_t em[4];
  float eb[4];
  auto load_ep = [&](int t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ej[j] = s_rows[(t - t_first) * RT + 16 * et + 4 * g + j];
      em[j] = tok_full[ej[j]];
      eb[j] = b_act ? b_act[ej[j]] : 0.f;
    }
  };
  // the end of tile t's segment [seg0, jend]: the W-wave sum, then the tile's epilogue
  // here or a published part
  auto flush = [&](int t, long long seg0, long long jend) {
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) s_acc[wave][i][m][tt][lane] = acc[i][m][tt];
    __syncthreads();
    if (wave < TR) {
      float4_t v[NM][NT];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          v[m][tt] = s_acc[0][et][m][tt][lane];
#pragma unroll
          for (int ww = 1; ww < W; ++ww) v[m][tt] += s_acc[ww][et][m][tt][lane];
        }
      const long long tb = (long long)t * KBT;
      bool fin = true;
      if (!(seg0 == tb && jend == tb + KBT - 1)) {
        float* pt = part + ((size_t)(2 * gi + (j0 >= tb ? 0 : 1)) * TR + et) * NO;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              __hip_atomic_store(pt + ((m * NT + tt) * 4 + c) * 64 + lane, v[m][tt][c],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int glo = owner_of(tb), np = owner_of(tb + KBT - 1) - glo + 1;
        int old = 0;
        if (lane == 0)
          old = __hip_atomic_fetch_add(tcnt + t * TR + et, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        fin = old == np - 1;
        if (fin) {
          asm volatile("" ::: "memory");
          // every part's loads first (parts past np repeat the last), then the sum in
          // workgroup order
          float pv[SK_PMAX][NM][NT][4];
#pragma unroll
          for (int q = 0; q < SK_PMAX; ++q) {
            const int gg = glo + min(q, np - 1);
            const float* pq = part + ((size_t)(2 * gg + (start_of(gg) >= tb ? 0 : 1)) * TR + et) * NO;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  pv[q][m][tt][c] = __hip_atomic_load(pq + ((m * NT + tt) * 4 + c) * 64 + lane,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                float a = pv[0][m][tt][c];
#pragma unroll
                for (int q = 1; q < SK_PMAX; ++q) a += q < np ? pv[q][m][tt][c] : 0.f;
                v[m][tt][c] = a;
              }
          if (lane == 0) __hip_atomic_store(tcnt + t * TR + et, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (fin) {
        if (r16 == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int p = t * RT + 16 * et + 4 * g + j;
            if (p < cnt) {
              idx[p] = ej[j];
              if (tokmask) tokmask[p] = em[j];
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const int b = tt * 16 + r16;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int p = t * RT + 16 * et + 4 * g + j;
            if (p < cnt && b < B) {
              const float a0 = v[0][tt][j] + eb[j];
              float h = a0 > 0.f ? a0 : 0.f;
              if (GATED) h *= v[NM - 1][tt][j];
              hT[(size_t)b * ldh + p] = ((em[j] >> b) & 1) ? h : 0.f;
            }
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[i][m][tt] = float4_t{0.f, 0.f, 0.f, 0.f};
  };
  long long j = j0, seg0 = j0;
  int t = t_first, kb = (int)(j0 - (long long)t_first * KBT);
  set_rows(t);
  load(2 * (kb * W + wave), 0);
  load_ep(t);
  while (true) {
    // block j: its first pair sits in buffer 0, its second goes to buffer 1
    load(2 * (kb * W + wave) + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mult(0);
    __builtin_amdgcn_sched_barrier(0);
    const long long jn = j + 1;
    const bool more = jn < j1;
    const bool next_tile = kb + 1 == KBT;
    const int kbn = next_tile ? 0 : kb + 1;
    if (more) {
      if (next_tile) set_rows(t + 1);
      load(2 * (kbn * W + wave), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mult(1);
    __builtin_amdgcn_sched_barrier(0);
    if (!more || next_tile) {
      flush(t, seg0, j);
      if (!more) break;
      t = t + 1;
      seg0 = jn;
      load_ep(t);
    }
    j = jn;
    kb = kbn;
  }
}

// Standalone token split (the forward entry point has no stage 1 to do it).
__global__ __launch_bounds__(TPB) void k_split_x(const float* __restrict__ x, int B, int d,
                                                 int tbp, u32x4* __restrict__ x_hl) {
  split_x_items(x, B, d, tbp, x_hl, blockIdx.x * TPB + threadIdx.x, gridDim.x * TPB);
}

// Down projection at batch: Y[b][c] += sum_p hT[b][p] * W_down^T[idx_p][c]. Workgroup
// (cb, kq) owns the 64-column block cb and list positions [p0, p1) (split kq of KS, a
// multiple of 32 positions each). Each wave streams its own 32-position chunks (chunk k of
// the split goes to wave k % 4): lane l reads row l/8 + 8j (j < 4) of the chunk, 16-byte
// piece l%8 of the block (whole 128-byte lines), stores the piece as is in the wave's own
// LDS buffer, and reads 8 consecutive positions of one column back as the right operand of
// v_mfma_f32_16x16x32_f16 with two LDS transpose reads (ds_read_b64_tr_b16: in each
// 16-lane group, lane i names position k0 + i / 4 at column n0 + 4 (i % 4), and lane j
// receives column n0 + j of positions k0 .. k0 + 3); the activations (token l%16, positions
// 8*(l/16)..+7) are the left one, as a hi + lo fp16 pair. No workgroup barrier in the
// loop; loads run one batch of KB chunks ahead. At the end the four waves' sums are added
// in wave order through LDS and leave as plain stores for KS == 1; else as float atomics
// onto y zeroed earlier in the call, or (JOIN) through the fixed-order join of the splits
// described at the single-token down projection, b_out riding on kq == 0.
constexpr int DCH = 32;         // positions per chunk (one k-step)
constexpr int IDX_CAP = 4096;   // list window held in LDS (a multiple of DCH)
template <int NT, bool JOIN>
__global__ __launch_bounds__(TPB) void k_down_mfma(const void* __restrict__ w_down_t, int ld_down,
                                                   const float* __restrict__ b_out,
                                                   const float* __restrict__ hT, int ldh, int d,
                                                   int n, int B, const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ count, int KS,
                                                   float* __restrict__ y,
                                                   float* __restrict__ dn_part,
                                                   int32_t* __restrict__ dn_cnt) {
  constexpr int KB = NT <= 2 ? 2 : 1;   // chunks per load batch
  // chunk buffer: [32 positions][64 columns] fp16 at a pitch of 34 words (the transpose
  // reads take 8-byte aligned addresses)
  constexpr int WP = 68;
  __shared__ __attribute__((aligned(16))) _Float16 s_wt[TPB / 64][KB][DCH * WP];
  __shared__ float4_t s_acc[TPB / 64][4][NT][64];
  __shared__ int32_t s_idx[IDX_CAP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;
  const int nch = d / 8;
  const int ncb = gridDim.x / KS;
  const int cb = blockIdx.x % ncb, kq = blockIdx.x / ncb;
  const int cnt = min(max(*count, 0), n);
  const int per = (((cnt + KS - 1) / KS) + DCH - 1) / DCH * DCH;
  const int p0 = min(cnt, kq * per), p1 = min(cnt, p0 + per);
  const u32x4* wcol = reinterpret_cast<const u32x4*>(w_down_t) + min(cb * 8 + lc, nch - 1);
  const float* hrow[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) hrow[tt] = hT + (size_t)min(16 * tt + r16, B - 1) * ldh;
  _Float16* swt = &s_wt[wave][0][0];

  float4_t acc[4][NT];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[cg][tt] = float4_t{0.f, 0.f, 0.f, 0.f};
  u32x4 wv[2][KB][4];
  float4_t av[2][KB][NT][2];
  int wb = p0, wl = 0;
  for (wb = p0; wb < p1; wb += IDX_CAP) {
    wl = min(IDX_CAP, p1 - wb);
    __syncthreads();
    // the list comes from the up kernel through the last-level cache: a batch of 8 entries
    // per thread is loaded before any is stored (entries past the window repeat its last
    // one, same value to the same place, so no store is conditional)
    for (int k0 = 0; k0 < wl; k0 += 8 * TPB) {
      int iv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) iv[j] = idx[wb + min(k0 + j * TPB + tid, wl - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) s_idx[min(k0 + j * TPB + tid, wl - 1)] = iv[j];
    }
    __syncthreads();
    const int nck = (wl + DCH - 1) / DCH;        // chunks in this window
    const int mine = (nck - wave + 3) / 4;       // this wave's chunks: wave, wave + 4, ...
    // window offset of this wave's chunk number i, clamped to its last chunk (a wave with
    // none reads chunk 0): every load stays within positions < wl + 31, inside the
    // activation row (rows are padded by 64 past the list's largest size) and the window's
    // indices; products of chunks past the end are skipped
    auto chunk_at = [&](int i) { return mine > 0 ? (wave + 4 * min(i, mine - 1)) * DCH : 0; };
    auto load = [&](int i0, int bb) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int pc = chunk_at(i0 + kb);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = s_idx[min(pc + lr + 8 * j, wl - 1)];
          wv[bb][kb][j] = ld_stream(wcol, (size_t)((i >= 0 && i < n) ? i : 0) * ld_down);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const float* hp = hrow[tt] + wb + pc + 8 * g;
          av[bb][kb][tt][0] = *reinterpret_cast<const float4_t*>(hp);
          av[bb][kb][tt][1] = *reinterpret_cast<const float4_t*>(hp + 4);
        }
      }
    };
    auto mult = [&](int i0, int bb) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        _Float16* bufk = swt + kb * DCH * WP;
        // stored as loaded: positions past the window end and invalid list entries meet
        // zero activations (the up projection writes 0 for invalid entries), columns past
        // d are never stored, so with finite weights they add nothing
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(bufk + (lr + 8 * j) * WP + 8 * lc);
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = wv[bb][kb][j][e];
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (i0 + kb < mine) {  // uniform within the wave
          const int pc = (wave + 4 * (i0 + kb)) * DCH;
          const _Float16* bufk = swt + kb * DCH * WP;
          half8_t ah[NT], al[NT];
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            float4_t v0 = av[bb][kb][tt][0], v1 = av[bb][kb][tt][1];
            const int q0 = pc + 8 * g;
            const bool tok = 16 * tt + r16 < B;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (!tok || q0 + e >= wl) v0[e] = 0.f;
              if (!tok || q0 + 4 + e >= wl) v1[e] = 0.f;
            }
            split_hi_lo(v0, v1, ah[tt], al[tt]);
          }
#pragma unroll
          for (int cg = 0; cg < 4; ++cg) {
            // positions 8g .. 8g + 7 of column 16 cg + r16
            const int col = 16 * cg + 4 * (r16 & 3), ra = 8 * g + (r16 >> 2);
            const short4_t ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4_t*)(bufk + ra * WP + col));
            const short4_t tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4_t*)(bufk + (ra + 4) * WP + col));
            const half8_t bw = __builtin_shufflevector(__builtin_bit_cast(half4_t, ta),
                                                       __builtin_bit_cast(half4_t, tb), 0, 1, 2, 3,
                                                       4, 5, 6, 7);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
              acc[cg][tt] = mfma16(ah[tt], bw, acc[cg][tt]);
              acc[cg][tt] = mfma16(al[tt], bw, acc[cg][tt]);
            }
          }
        }
      }
      wave_lds_sync();
    };
    // whole iterations while chunks remain past the next two batches; then the last one
    // or two batches with nothing fetched beyond the wave's own chunks (a wave retires only
    // when its loads have landed)
    load(0, 0);
    int i0 = 0;
    for (; i0 + 2 * KB < mine; i0 += 2 * KB) {
      load(i0 + KB, 1);
      __builtin_amdgcn_sched_barrier(0);
      mult(i0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load(i0 + 2 * KB, 0);
      __builtin_amdgcn_sched_barrier(0);
      mult(i0 + KB, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i0 + KB < mine) {  // uniform within the wave
      load(i0 + KB, 1);
      __builtin_amdgcn_sched_barrier(0);
      mult(i0, 0);
      __builtin_amdgcn_sched_barrier(0);
      mult(i0 + KB, 1);
    } else {
      mult(i0, 0);
    }
  }
  // fixed-order sum of the four waves, then out (lane l holds column 16cg + l%16 of the
  // block, tokens 16tt + 4*(l/16) + j)
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) s_acc[wave][cg][tt][lane] = acc[cg][tt];
  __syncthreads();
  if (JOIN && KS > 1) {
    // every split takes part, an empty one with zeros; slot o of split kq holds output o
    // The slots are written and read 16 bytes a lane with the device-coherent cache policy
    // (sc1, as agent-scope atomic stores and loads use), so every store fills whole lines:
    // one 4-byte coherent store per value would write each line through four times.
    constexpr int NO = 4 * NT * 64;
    __shared__ int s_last;
    float* slot = dn_part + (size_t)cb * KS * NO * 4;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(slot, 0, KS * NO * 16, BUF_RSRC_WORD3);
    float4_t mine[NT];
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const int o = it * TPB + tid;
      const int cg = o / (NT * 64), tt = (o / 64) % NT, l = o % 64;
      const int col = cb * 64 + 16 * cg + (l & 15);
      const float bo = (kq == 0 && b_out && col < d) ? b_out[col] : 0.f;
      mine[it] = ((s_acc[0][cg][tt][l] + s_acc[1][cg][tt][l]) + s_acc[2][cg][tt][l]) +
                 s_acc[3][cg][tt][l];
#pragma unroll
      for (int j = 0; j < 4; ++j) mine[it][j] += bo;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, mine[it]), rsrc,
                                             (kq * NO + o) * 16, 0, CPOL_SC1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(dn_cnt + cb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == KS - 1;
    __syncthreads();
    if (s_last) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        const int o = it * TPB + tid;
        const int cg = o / (NT * 64), tt = (o / 64) % NT, l = o % 64;
        const int col = cb * 64 + 16 * cg + (l & 15);
        float4_t pv[KS_JOIN_MAX];
#pragma unroll
        for (int q = 0; q < KS_JOIN_MAX; ++q) {
          if (q < KS && q != kq)
            pv[q] = __builtin_bit_cast(
                float4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (q * NO + o) * 16, 0, CPOL_SC1));
          else
            pv[q] = mine[it];
        }
        float4_t a = pv[0];
#pragma unroll
        for (int q = 1; q < KS_JOIN_MAX; ++q)
          if (q < KS) a += pv[q];
        if (col < d) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int b = 16 * tt + 4 * (l >> 4) + j;
            if (b < B) y[(size_t)b * d + col] = a[j];
          }
        }
      }
      if (tid == 0) __hip_atomic_store(dn_cnt + cb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (kq == 0 || p1 > p0) {
    // 4 * NT * 64 outputs, NT per thread: a fixed trip count, so the b_out loads of all
    // of them go out together
    static_assert(4 * 64 == TPB, "one output per thread and token tile");
    float bo[NT];
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const int o = it * TPB + tid;
      const int col = cb * 64 + 16 * (o / (NT * 64)) + (o & 15);
      bo[it] = (kq == 0 && b_out && col < d) ? b_out[col] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const int o = it * TPB + tid;
      const int cg = o / (NT * 64), tt = (o / 64) % NT, l = o % 64;
      const float4_t v = ((s_acc[0][cg][tt][l] + s_acc[1][cg][tt][l]) + s_acc[2][cg][tt][l]) +
                         s_acc[3][cg][tt][l];
      const int col = cb * 64 + 16 * cg + (l & 15);
      if (col < d) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int b = 16 * tt + 4 * (l >> 4) + j;
          if (b < B) {
            float* dst = y + (size_t)b * d + col;
            if (KS == 1)
              *dst = v[j] + bo[it];
            else
              atomicAdd(dst, v[j] + bo[it]);
          }
        }
      }
    }
  }
}

template <bool F16>
hipError_t scores_launch(const LayerDev& L, int B, float* scores, hipStream_t s) {
  const int nchp = L.r / (F16 ? 8 : 4);
  int Lw, cplp;
  pick_group(nchp, Lw, cplp);
  constexpr int PASSES = 4;
  const int rows_per_wg = (TPB / Lw) * PASSES;
  const dim3 grid((L.n + rows_per_wg - 1) / rows_per_wg);
#define SCORES(LL, CC)                                                                       \
  hipLaunchKernelGGL((k_pred_scores<F16, LL, CC, PASSES>), grid, dim3(TPB), 0, s, L.p2,      \
                     L.p_bias, L.q, L.n, L.r, B, scores)
  if (Lw == 8) SCORES(8, 1);
  else if (Lw == 16) SCORES(16, 1);
  else if (Lw == 32) SCORES(32, 1);
  else if (cplp == 1) SCORES(64, 1);
  else if (cplp == 2) SCORES(64, 2);
  else SCORES(64, 4);
#undef SCORES
  return hipGetLastError();
}

// fw: the up kernel lists the union itself from the words and token bits the score kernel
// left in the workspace, writing idx, count and tokmask; otherwise it reads them
template <bool GATED, int NT, int TR, int W, bool HALF = false>
void up_tile_launch_t(const LayerDev& L, int B, const int32_t* idx, const int32_t* count,
                      const uint64_t* tokmask, const uint64_t* tok_by_neuron, float* y0, int ny,
                      hipStream_t s, const hipEvent_t* tev, bool fw) {
  int32_t* idx_w = const_cast<int32_t*>(idx);
  int32_t* cnt_w = const_cast<int32_t*>(count);
  uint64_t* tok_w = const_cast<uint64_t*>(tokmask);
  if (fw)
    launch(k_up_mfma<GATED, NT, TR, W, true, HALF>, dim3(L.g_up), dim3(64 * W), 0, s, tev, L.w_act, L.act_ld,
           L.b_act, static_cast<const u32x4*>(L.x_hl), L.d, L.n, B, idx_w, cnt_w, tok_w,
           (const uint64_t*)L.words, (const uint64_t*)L.tok_full, L.h_buf, L.ldh, y0, ny);
  else
    launch(k_up_mfma<GATED, NT, TR, W, false, HALF>, dim3(L.g_up), dim3(64 * W), 0, s, tev, L.w_act, L.act_ld,
           L.b_act, static_cast<const u32x4*>(L.x_hl), L.d, L.n, B, idx_w, cnt_w, tok_w,
           (const uint64_t*)nullptr, tok_by_neuron, L.h_buf, L.ldh, y0, ny);
}

// At 16 tokens (one token tile) each workgroup takes two row tiles with eight waves
// splitting d, so each activation fragment serves both tiles and the pairs stay about as
// many as the compute units. Otherwise one row tile and four waves: with two token tiles a
// paired workgroup needs more registers than let two of them share a compute unit, and
// the pairs then outnumber the compute units (measured no faster at 32 tokens); below 16
// tokens eight waves on one row tile measured slower (2 tokens 18.3 vs 17.5 us, 8 tokens
// 30.9 vs 26.7 us on the Llama-7B shape). Up to L.up_half_b tokens (a union expected to
// fill at most half the compute units with 16-row tiles) a tile takes 8 listed rows.
template <bool GATED, int NT, int TR, int W>
void up_sk_launch(const LayerDev& L, int B, int32_t* idx, int32_t* count, uint64_t* tokmask,
                  float* y0, int ny, hipStream_t s, const hipEvent_t* tev, int grid) {
  launch(k_up_sk<GATED, NT, TR, W>, dim3(grid), dim3(64 * W), 0, s, tev, L.w_act, L.act_ld, L.b_act,
         static_cast<const u32x4*>(L.x_hl), L.d, L.n, B, idx, count, tokmask,
         (const uint64_t*)L.words, (const uint64_t*)L.tok_full, L.h_buf, L.ldh, y0, ny,
         L.sk_part, L.sk_cnt);
}

// The stream-K form runs at 17-32 tokens (the decode step's list from the words): one row
// tile, four waves, two workgroups per compute unit (g_sk); d a multiple of 512 with at
// least two input blocks per tile, and ranges that touch at most SK_TMAX tiles (g_sk >=
// tiles / 13). Measured on the Llama-7B-shaped gated stack it gains at 32 tokens (82.9 vs
// 84.4 us a layer); wherever the ranges are only a few blocks long the hand-offs (about a
// coherent round trip each) cost more than the balance gains:
//  - 4 tokens, one row tile: 35.3 vs 33.1 us (every tile split);
//  - 16 tokens, one row tile: 55.2 vs 51.0 us (the two-row-tile eight-wave kernel shares
//    each activation fragment between two row tiles);
//  - 16 tokens, two row tiles and eight waves on all 256 compute units instead of 197:
//    54.0 vs 51.4 us (about 3 blocks per range, so almost every tile is split).
int up_sk_form(const LayerDev& L, int B, bool fw) {
  if (!fw || !L.sk_part) return 0;
  if (B > 16 && B <= 32 && L.d % 512 == 0 && L.d >= 1024 && L.g_sk * 13 >= (L.n + 15) / 16)
    return 1;
  return 0;
}

template <bool GATED>
void up_tile_launch(const LayerDev& L, int B, const int32_t* idx, const int32_t* count,
                    const uint64_t* tokmask, const uint64_t* tok_by_neuron, float* y0, int ny,
                    hipStream_t s, const hipEvent_t* tev, bool fw) {
  const int nt = (B + 15) / 16;
  if (up_sk_form(L, B, fw) != 0) {
    int32_t* idx_w = const_cast<int32_t*>(idx);
    int32_t* cnt_w = const_cast<int32_t*>(count);
    uint64_t* tok_w = const_cast<uint64_t*>(tokmask);
    up_sk_launch<GATED, 2, 1, 4>(L, B, idx_w, cnt_w, tok_w, y0, ny, s, tev, L.g_sk);
    return;
  }
  if (B >= 16 && nt == 1 && L.d % 512 == 0) {
    up_tile_launch_t<GATED, 1, 2, 8>(L, B, idx, count, tokmask, tok_by_neuron, y0, ny, s, tev, fw);
    return;
  }
  switch (nt) {
    case 1:
      if (B <= L.up_half_b)
        up_tile_launch_t<GATED, 1, 1, 4, true>(L, B, idx, count, tokmask, tok_by_neuron, y0, ny, s, tev, fw);
      else
        up_tile_launch_t<GATED, 1, 1, 4>(L, B, idx, count, tokmask, tok_by_neuron, y0, ny, s, tev, fw);
      break;
    case 2: up_tile_launch_t<GATED, 2, 1, 4>(L, B, idx, count, tokmask, tok_by_neuron, y0, ny, s, tev, fw); break;
    case 3: up_tile_launch_t<GATED, 3, 1, 4>(L, B, idx, count, tokmask, tok_by_neuron, y0, ny, s, tev, fw); break;
    default: up_tile_launch_t<GATED, 4, 1, 4>(L, B, idx, count, tokmask, tok_by_neuron, y0, ny, s, tev, fw); break;
  }
}

template <int NT>
void down_tile_launch_t(const LayerDev& L, int B, const int32_t* idx, const int32_t* count,
                        float* y, hipStream_t s, const hipEvent_t* tev) {
  const dim3 grid(((L.d + 63) / 64) * L.ks_tile);
  if (L.join_tile)
    launch(k_down_mfma<NT, true>, grid, dim3(TPB), 0, s, tev, L.w_down_t, L.down_ld, L.b_out,
           L.h_buf, L.ldh, L.d, L.n, B, idx, count, L.ks_tile, y, L.dn_part, L.dn_cnt);
  else
    launch(k_down_mfma<NT, false>, grid, dim3(TPB), 0, s, tev, L.w_down_t, L.down_ld, L.b_out,
           L.h_buf, L.ldh, L.d, L.n, B, idx, count, L.ks_tile, y, nullptr, nullptr);
}

void down_tile_launch(const LayerDev& L, int B, const int32_t* idx, const int32_t* count,
                      float* y, hipStream_t s, const hipEvent_t* tev) {
  switch ((B + 15) / 16) {
    case 1: down_tile_launch_t<1>(L, B, idx, count, y, s, tev); break;
    case 2: down_tile_launch_t<2>(L, B, idx, count, y, s, tev); break;
    case 3: down_tile_launch_t<3>(L, B, idx, count, y, s, tev); break;
    default: down_tile_launch_t<4>(L, B, idx, count, y, s, tev); break;
  }
}

// union-list forward on the matrix cores; y is zeroed by the up kernel when the down
// projection splits rows. Standalone (zero_y) the tokens are split here; in the decode
// step stage 1 has split them.
void forward_tiles(const LayerDev& L, const float* x, int B, const int32_t* idx,
                   const int32_t* count, const uint64_t* tokmask, const uint64_t* tok_by_neuron,
                   float* y, bool zero_y, bool fw, hipStream_t s, const hipEvent_t* t_up,
                   const hipEvent_t* t_down) {
  const int ny = (zero_y && L.ks_tile > 1 && !L.join_tile) ? B * L.d : 0;
  if (zero_y) {
    const int items = L.d / 8 * B;
    hipLaunchKernelGGL(k_split_x, dim3((items + TPB - 1) / TPB), dim3(TPB), 0, s, x, B, L.d, B,
                       static_cast<u32x4*>(L.x_hl));
  }
  if (L.gated)
    up_tile_launch<true>(L, B, idx, count, tokmask, tok_by_neuron, y, ny, s, t_up, fw);
  else
    up_tile_launch<false>(L, B, idx, count, tokmask, tok_by_neuron, y, ny, s, t_up, fw);
  down_tile_launch(L, B, idx, count, y, s, t_down);
}

}  // namespace

hipError_t run_scores(const LayerDev& L, int B, float* scores, hipStream_t s) {
  return L.p_f16 ? scores_launch<true>(L, B, scores, s) : scores_launch<false>(L, B, scores, s);
}

hipError_t launch_compact(const LayerDev& L, const float* scores, int B, int32_t* idx,
                          int32_t* count, uint64_t* tokmask, hipStream_t s) {
  hipLaunchKernelGGL(k_cmp_tiles, dim3(L.n_tiles), dim3(TPB), 0, s, scores, L.n, B, L.tau,
                     L.tok_full, L.words);
  hipLaunchKernelGGL(k_cmp_scatter, dim3(L.n_tiles), dim3(TPB), 0, s, L.tok_full, L.words, L.n,
                     L.n_tiles, idx, count, tokmask);
  return hipGetLastError();
}

static size_t score_tiles_lds(const LayerDev& L, int B) {
  const int nt = (B + 15) / 16;
  return (size_t)L.r * ((16 * nt + 31) / 32 * 32) * 4;
}

bool score_tiles_ok(const LayerDev& L, int B) {
  const int epc = L.p_f16 ? 8 : 4;
  return B >= 1 && B <= MAXB && L.r % (4 * epc) == 0 && score_tiles_lds(L, B) <= SCORE_Q_LDS;
}

hipError_t run_score_tiles(const LayerDev& L, int B, float* scores, hipStream_t s) {
  const dim3 grid((L.n + 63) / 64);
  const size_t lds = score_tiles_lds(L, B);
#define SFFN_ST(F16, NT)                                                                     \
  hipLaunchKernelGGL((k_score_tiles<F16, NT>), grid, dim3(TPB), lds, s, L.p2, L.p_bias, L.q, \
                     L.n, L.r, B, L.tau, L.tok_full, L.words, scores)
  const int nt = (B + 15) / 16;
  if (L.p_f16) {
    if (nt == 1) SFFN_ST(true, 1); else if (nt == 2) SFFN_ST(true, 2);
    else if (nt == 3) SFFN_ST(true, 3); else SFFN_ST(true, 4);
  } else {
    if (nt == 1) SFFN_ST(false, 1); else if (nt == 2) SFFN_ST(false, 2);
    else if (nt == 3) SFFN_ST(false, 3); else SFFN_ST(false, 4);
  }
#undef SFFN_ST
  return hipGetLastError();
}

hipError_t launch_scatter(const LayerDev& L, int32_t* idx, int32_t* count, uint64_t* tokmask,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_cmp_scatter, dim3(L.n_tiles), dim3(TPB), 0, s, L.tok_full, L.words, L.n,
                     L.n_tiles, idx, count, tokmask);
  return hipGetLastError();
}

bool union_in_up_ok(const LayerDev& L) { return (L.n + 63) / 64 <= FW_WORDS_MAX; }

void run_forward_tiles(const LayerDev& L, const float* x, int B, const int32_t* idx,
                       const int32_t* count, const uint64_t* tokmask,
                       const uint64_t* tok_by_neuron, float* y, bool zero_y, bool from_words,
                       hipStream_t s, const hipEvent_t* t_up, const hipEvent_t* t_down) {
  forward_tiles(L, x, B, idx, count, tokmask, tok_by_neuron, y, zero_y, from_words, s, t_up,
                t_down);
}

}  // namespace sffn
