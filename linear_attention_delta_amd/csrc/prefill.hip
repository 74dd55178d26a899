// prefill.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The oxydllm 0.0.0-alpha.12.2 release notes ("New Features", Gated DeltaNet
// runtime; "Performance", Gated DeltaNet fast paths) run prefill as a chunked
// parallel scan: the state-independent work of every chunk is done in batch,
// then a sequential loop carries the state across chunks.  For a chunk of C
// tokens (gamma_r = g_0 + ... + g_r inside the chunk, k_hat = rk k,
// q_hat = rq q, rk = 1/|k|, rq = scale/|q|):
//
//   A[r,s] = beta_r e^{gamma_r - gamma_s} k_hat_r . k_hat_s     (s < r)
//   Tt     = (I + A)^{-1} diag(beta)
//   P[r,s] = e^{gamma_r - gamma_s} q_hat_r . k_hat_s          (s <= r)
//   a_r = e^{gamma_r} rk_r,  b_r = e^{gamma_r} rq_r,  c_r = e^{gamma_last - gamma_r} rk_r
//
//   U  = Tt (V - diag(a) K S)                                -- new values
//   O  = diag(b) Q S + P U
//   S <- e^{gamma_last} S + K^T diag(c) U
//
// Phase 1 (k_prepare): one workgroup per (chunk, q/k head, pair of v-heads),
// fully parallel.  It forms K K^T and K Q^T on the matrix cores, inverts
// I + A blockwise --
// the doubling product (I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8) on each 16x16
// diagonal block (N^16 = 0), then pairwise merging 16 -> 32 -> 64 with
// [[X,0],[Y,Z]]^{-1} = [[X^-1,0],[-Z^-1 Y X^-1, Z^-1]] -- never powers of the
// whole 64x64 block, which overflow fp32 on repeated tokens (the notes'
// failure of plain doubling at chunk 64) -- and writes Tt, P and a, b, c,
// e^{gamma_last} to the workspace.
//
// Phase 2 (k_scan): one workgroup per (sequence, v-head, NT*16 columns of
// d_v) walks the chunks in order with its d_k x NT*16 fp32 slice of S in
// registers; per chunk only the four state-dependent products remain.
#include <algorithm>
#include <type_traits>

#include "gate_math.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr float kL2Eps = 1e-6f;

// ------------------------------------------------------------ chunk table
// chunk_offsets[i] = sum_{j<i} ceil(len_j / C), and for the segment-parallel
// path seg_offsets[i] = sum_{j<i} max(1, ceil(ceil(len_j / C) / seg_len)).
// One workgroup; sequential over blocks of 1024 sequences, scan inside a block.
__global__ void __launch_bounds__(1024) k_chunk_table(ScanArgs a) {
  __shared__ int carry[2];
  __shared__ int buf[2][1024];
  if (threadIdx.x < 2) carry[threadIdx.x] = 0;
  __syncthreads();
  for (int base = 0; base < a.num_seqs; base += 1024) {
    const int i = base + threadIdx.x;
    int n = 0, ns = 0;
    if (i < a.num_seqs) {
      const int len = a.cu_seqlens[i + 1] - a.cu_seqlens[i];
      n = (len + a.chunk - 1) / a.chunk;
      if (a.seg_offsets) ns = n > 0 ? (n + a.seg_len - 1) / a.seg_len : 1;
    }
    buf[0][threadIdx.x] = n;
    buf[1][threadIdx.x] = ns;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scans
      const int v0 = threadIdx.x >= off ? buf[0][threadIdx.x - off] : 0;
      const int v1 = threadIdx.x >= off ? buf[1][threadIdx.x - off] : 0;
      __syncthreads();
      buf[0][threadIdx.x] += v0;
      buf[1][threadIdx.x] += v1;
      __syncthreads();
    }
    if (i < a.num_seqs) {
      a.chunk_offsets[i + 1] = carry[0] + buf[0][threadIdx.x];
      if (a.seg_offsets) a.seg_offsets[i + 1] = carry[1] + buf[1][threadIdx.x];
    }
    __syncthreads();
    if (threadIdx.x == 1023) {
      carry[0] += buf[0][1023];
      carry[1] += buf[1][1023];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.chunk_offsets[0] = 0;
    if (a.seg_offsets) a.seg_offsets[0] = 0;
  }
  // The carry's dispatch order: its units (segments on the segment path,
  // else sequences) by chunk count, longest first (ties by index), so the
  // longest chains start in the first round of workgroups.  A rank sort,
  // one unit per thread, up to 1024 units; past that the identity.  Only
  // the order changes, not what any workgroup computes.
  if (a.seg_perm) {
    __shared__ int slen[1024];
    const bool segs = a.seg_offsets != nullptr;
    const int total = segs ? carry[1] : a.num_seqs;
    if (total <= 1024) {
      // then num_seqs <= 1024 (a sequence has at least one segment): the loop
      // above ran once, and buf[1][i] is sequence i's inclusive segment count
      const int i = threadIdx.x;
      if (i < a.num_seqs) {
        const int len = a.cu_seqlens[i + 1] - a.cu_seqlens[i];
        const int n = (len + a.chunk - 1) / a.chunk;
        if (segs) {
          const int ns = n > 0 ? (n + a.seg_len - 1) / a.seg_len : 1;
          const int first = buf[1][i] - ns;
          for (int p = 0; p < ns; p++) slen[first + p] = min(a.seg_len, n - p * a.seg_len);  // 0: empty sequence
        } else {
          slen[i] = n;
        }
      }
      __syncthreads();
      const int t = threadIdx.x;
      if (t < total) {
        const int lt = slen[t];
        int rank = 0;
        for (int u = 0; u < total; u++) {
          const int lu = slen[u];
          rank += (lu > lt) || (lu == lt && u < t);
        }
        a.seg_perm[rank] = t;
      }
    } else {
      for (int t = threadIdx.x; t < total; t += 1024) a.seg_perm[t] = t;
    }
  }
}

// Locate global chunk n: its sequence, first token and length.  false if
// n is past the last chunk (varlen grids are sized by an upper bound).
__device__ __forceinline__ bool chunk_of(const ScanArgs& a, int C, int n, int& seq, int& start, int& len) {
  if (a.seqlen > 0) {
    const int cps = (a.seqlen + C - 1) / C;
    seq = n / cps;
    if (seq >= a.num_seqs) return false;
    const int c = n - seq * cps;
    start = seq * a.seqlen + c * C;
    len = min(C, a.seqlen - c * C);
    return true;
  }
  if (n >= a.chunk_offsets[a.num_seqs]) return false;
  int lo = 0, hi = a.num_seqs - 1;  // last seq with offsets[seq] <= n
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.chunk_offsets[mid] <= n) lo = mid; else hi = mid - 1;
  }
  seq = lo;
  start = a.cu_seqlens[seq] + (n - a.chunk_offsets[seq]) * C;
  len = min(C, a.cu_seqlens[seq + 1] - start);
  return true;
}

// Inclusive prefix sum of one value per lane over the first n lanes of a
// wave (lanes >= n contribute their value too; callers pass 0 there).
__device__ __forceinline__ float wave_prefix_sum(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// ----------------------------------------------- fp32 16x16 tile products
// D = A(16 x K) B(K x 16), A and B row-major in LDS (fp32 matrix cores).
template <int K>
__device__ __forceinline__ f32x4 mm16_f32(const float* A, int lda, const float* B, int ldb, int lane) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < K; kb += 4)
    acc = mfma16(A[r * lda + kb + q], B[(kb + q) * ldb + r], acc);
  return acc;
}

__device__ __forceinline__ void st16(float* D, int ldd, f32x4 v, int lane) {
  const int c = lane & 15, r0 = (lane >> 4) * 4;
#pragma unroll
  for (int e = 0; e < 4; e++) D[(r0 + e) * ldd + c] = v[e];
}

// Same, adding the identity (D = I + v).
__device__ __forceinline__ void st16_plus_i(float* D, int ldd, f32x4 v, int lane) {
  const int c = lane & 15, r0 = (lane >> 4) * 4;
#pragma unroll
  for (int e = 0; e < 4; e++) D[(r0 + e) * ldd + c] = v[e] + (r0 + e == c ? 1.f : 0.f);
}

// ---------------------------------------------------------------- phase 1
//
// One workgroup per (chunk, q/k head, HPW of the v-heads that read it): K
// and Q are staged once, the raw products K K^T and Q K^T are formed once
// on the matrix cores and scaled per v-head (the decays and beta are per
// v-head).  The chunk inverse runs in registers on 16x16 fp32 tiles held in
// the accumulator layout (lane (c, g) holds T[4g+e][c]); a product X Y is
// four 16x16x4 steps whose k index runs over {4g + t}, so its operands are
// X^T and Y in that same layout and no lane exchange is needed.
// Workspace block of one (chunk, v-head): Tt [C][C] then P [C][C] in the
// operand type, and (separately) 4 x C fp32 scalars: a, b, c and
// e^{gamma_last} (first element of the fourth row).

template <class E, int C, int DK, int HPW>
struct alignas(16) PrepSmem {
  typedef typename E::store_t T;
  static constexpr int KLD = DK + 16 / sizeof(T);  // row pad: 16 bytes
  static constexpr int ALD = C + 4;                // 16-byte aligned rows
  union U {
    struct { T k[C][KLD]; T q[C][KLD]; } in;       // Gram operands
    float at[HPW][C][ALD];                         // A per v-head, then its inverse in place
  } u;
  float gam[HPW][C], bet[HPW][C], rk[C], rq[C];
};



// X Y for 16x16 fp32 tiles given X^T and Y in the accumulator layout.
__device__ __forceinline__ f32x4 mm_tt(f32x4 xt, f32x4 y) {
  f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; t++) d = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[t], y[t], d, 0, 0, 0);
  return d;
}

// 16x16 tile of a row-major fp32 array (leading dimension L) in the
// accumulator layout, as itself (ld_c) or transposed (ld_ct).
__device__ __forceinline__ f32x4 ld_c(const float* M, int L, int lane) {
  const int c = lane & 15, g = lane >> 4;
  return f32x4{M[(4 * g) * L + c], M[(4 * g + 1) * L + c], M[(4 * g + 2) * L + c], M[(4 * g + 3) * L + c]};
}
__device__ __forceinline__ f32x4 ld_ct(const float* M, int L, int lane) {
  return *reinterpret_cast<const f32x4*>(M + (lane & 15) * L + 4 * (lane >> 4));
}
__device__ __forceinline__ void st_c(float* M, int L, f32x4 v, int lane) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int e = 0; e < 4; e++) M[(4 * g + e) * L + c] = v[e];
}
__device__ __forceinline__ f32x4 ident_c(int lane) {
  const int c = lane & 15, g = lane >> 4;
  return f32x4{4 * g == c ? 1.f : 0.f, 4 * g + 1 == c ? 1.f : 0.f, 4 * g + 2 == c ? 1.f : 0.f,
               4 * g + 3 == c ? 1.f : 0.f};
}

// Transpose of a 16x16 tile in the accumulator layout through the wave's own
// 16x16 LDS block at T0 (leading dimension L): written, then read back
// transposed.  One wave's LDS operations complete in order; the wait and the
// memory clobber keep the compiler from moving the read above the writes.
__device__ __forceinline__ f32x4 transpose_lds(float* T0, int L, f32x4 v, int lane) {
  st_c(T0, L, v, lane);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const f32x4 t = ld_ct(T0, L, lane);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  return t;
}

// (I + N)^{-1} of a strictly lower 16x16 block N (row-major at A0) by the
// doubling product (I - N)(I + N^2)(I + N^4)(I + N^8), N^16 = 0.  The
// factors are polynomials in N and commute, so each step multiplies from the
// side whose transpose is at hand; the transposes of N^2 and N^4 go through
// the block's own LDS (free once N is in registers) instead of two more
// products.  The caller writes the inverse back over A0.
__device__ __forceinline__ f32x4 inv16(float* A0, int L, int lane) {
  const f32x4 id = ident_c(lane);
  const f32x4 n = ld_c(A0, L, lane), nt = ld_ct(A0, L, lane);
  const f32x4 n2 = mm_tt(nt, n);
  const f32x4 n2t = transpose_lds(A0, L, n2, lane);
  const f32x4 n4 = mm_tt(n2t, n2);
  const f32x4 n4t = transpose_lds(A0, L, n4, lane);
  const f32x4 n8t = mm_tt(n4, n4t);
  const f32x4 x1 = mm_tt(id - nt, id + n2);   // (I - N)(I + N^2)
  const f32x4 x2 = mm_tt(id + n4t, x1);       // (I + N^4) x1
  return mm_tt(id + n8t, x2);                 // (I + N^8) x2
}

// Waves per prepare workgroup.
constexpr int kPrepWaves = 8;

// WQ: also stage Q and write P and b (what the sequential carry reads); the
// segment-parallel carry forms P itself from Q and K, so without WQ only K
// is read and P is not written.
template <class E, int C, int DK, int HPW, bool WQ>
__global__ void __launch_bounds__(64 * kPrepWaves) k_prepare(ScanArgs a) {
  constexpr int PW = kPrepWaves, PT = 64 * kPrepWaves;
  typedef typename E::store_t T;
  typedef PrepSmem<E, C, DK, HPW> SM;
  constexpr int NRT = C / 16;
  constexpr int NT = NRT * (NRT + 1) / 2;      // lower 16x16 tiles (diagonal included)
  constexpr int NTW = (NT + PW - 1) / PW;      // per wave
  constexpr int L = SM::ALD;
  __shared__ SM sm;
  // one-dimensional grid: workgroup = (chunk, q/k head with HPW of its v-heads)
  const int G = a.hv / a.hk;
  const int ngroups = a.hv / HPW;
  const long chunk = blockIdx.x / ngroups;
  const int grp = blockIdx.x % ngroups;
  int seq, start, len;
  if (!chunk_of(a, C, (int)chunk, seq, start, len)) return;
  const int hk = grp / (G / HPW);
  const int vh0 = (grp % (G / HPW)) * HPW;
  int hs[HPW];
#pragma unroll
  for (int j = 0; j < HPW; j++) hs[j] = a.tiled ? (hk + (vh0 + j) * a.hk) : (hk * G + vh0 + j);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int c16 = lane & 15, r4 = (lane >> 4) * 4;

  // ---- load K and Q rows (zero past the end of the sequence) and the
  // gates; all loads are issued before any is used.  Rows and lanes outside
  // the chunk read a clamped, valid address and are masked afterwards: a
  // load inside a branch makes the compiler drain every load in flight
  // where the branch rejoins (one more memory round trip each).
  constexpr int EPV = 16 / sizeof(T);
  constexpr int VPR = DK / EPV;  // 16-byte vectors per row
  constexpr int KQV = (WQ ? 2 : 1) * C * VPR;    // 16-byte vectors of K (and Q)
  constexpr int NV = (KQV + PT - 1) / PT;
  u32x4 w[NV];
  {
    const T* kp = reinterpret_cast<const T*>(a.k);
    const T* qp = reinterpret_cast<const T*>(a.q);
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int idx = tid + PT * j;
      const int which = idx / (C * VPR);
      const int rem = idx % (C * VPR);
      const int r = rem / VPR, cv = rem % VPR;
      const int rr = min(r, len - 1);
      if (KQV % PT == 0 || idx < KQV) {
        const T* src = which ? qp + (long)(start + rr) * a.stride_q : kp + (long)(start + rr) * a.stride_k;
        w[j] = *reinterpret_cast<const u32x4*>(src + (long)hk * DK + cv * EPV);
        if (r >= len) w[j] = u32x4{0u, 0u, 0u, 0u};
      } else {
        w[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  float gv = 0.f, bv = 0.f;
  if (a.gate_a) {
    if (wave < HPW && lane < len) gates_from_raw<E>(a, start + lane, hs[wave], gv, bv);
  } else {
    const bool mine = wave < HPW && lane < len;
    const long gi = (long)(start + min(lane, len - 1)) * a.hv + hs[wave < HPW ? wave : 0];
    gv = mine ? a.g[gi] : 0.f;
    bv = mine ? a.beta[gi] : 0.f;
  }

  // ---- stage K and Q into LDS with the per-row inverse norms
  {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int idx = tid + PT * j;
      const int which = idx / (C * VPR);
      const int rem = idx % (C * VPR);
      const int r = rem / VPR, cv = rem % VPR;
      if (idx < KQV) *reinterpret_cast<u32x4*>(which ? &sm.u.in.q[r][cv * EPV] : &sm.u.in.k[r][cv * EPV]) = w[j];
      float ss = 0.f;
      if constexpr (std::is_same<E, BF16>::value) {
#pragma unroll
        for (int i = 0; i < 4; i++) ss = dot2_bf16(w[j][i], w[j][i], ss);
      } else {
        const T* e = reinterpret_cast<const T*>(&w[j]);
#pragma unroll
        for (int i = 0; i < EPV; i++) {
          const float x = E::to_f32(e[i]);
          ss += x * x;
        }
      }
      ss = group_sum<VPR>(ss);
      if (cv == 0 && idx < KQV) {
        const float inv = a.l2norm ? __builtin_amdgcn_rsqf(ss + kL2Eps) : 1.0f;
        if (which) sm.rq[r] = a.scale * inv; else sm.rk[r] = inv;
      }
    }
  }
  if (wave < HPW) {
    const float gm = wave_prefix_sum(gv, lane);
    if (lane < C) {
      sm.gam[wave][lane] = gm;
      sm.bet[wave][lane] = bv;
    }
  }
  lds_barrier();
  // ---- transposed Gram tiles D[s][r] = k_s . x_r (x = k or q) of the lower
  // tile (i, j), j <= i: lane (c, g) holds r = 16i + c, s = 16j + 4g + e.
  //   P[r][s] = rq_r rk_s e^{gamma_r - gamma_s} q_r.k_s          (s <= r) -> workspace
  //   A[r][s] = beta_r rk_r rk_s e^{gamma_r - gamma_s} k_r.k_s   (s < r)  -> registers, then LDS
  auto tile_ij = [](int t, int& i, int& j) {
    i = 0;
    while ((i + 1) * (i + 2) / 2 <= t) i++;
    j = t - i * (i + 1) / 2;
  };
  f32x4 rawA[NTW];
#pragma unroll
  for (int n = 0; n < NTW; n++) {
    const int t = wave + PW * n;
    if (t < NT) {
      int i, j;
      tile_ij(t, i, j);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      rawA[n] = tile_mma<E, DK>(acc, &sm.u.in.k[16 * j][0], SM::KLD, &sm.u.in.k[16 * i][0], SM::KLD, lane);
    }
  }
  if constexpr (WQ) {
  for (int t = wave; t < NT; t += PW) {
    int i, j;
    tile_ij(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile_mma<E, DK>(acc, &sm.u.in.k[16 * j][0], SM::KLD, &sm.u.in.q[16 * i][0], SM::KLD, lane);
    const int r = 16 * i + c16, s0 = 16 * j + r4;
    const float fr = sm.rq[r];
    const f32x4 rks = *reinterpret_cast<const f32x4*>(&sm.rk[s0]);
#pragma unroll
    for (int hh = 0; hh < HPW; hh++) {
      const float gr = sm.gam[hh][r];
      const f32x4 gs = *reinterpret_cast<const f32x4*>(&sm.gam[hh][s0]);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        // computed for every element, then selected (a masked one may be inf)
        const float val = fr * rks[e] * __expf(gr - gs[e]) * acc[e];
        v[e] = s0 + e <= r ? val : 0.f;
      }
      // packed like Tt: lower block t (row-major, 256 values) at 256 t
      T* pout = reinterpret_cast<T*>(a.tinv) + (chunk * a.hv + hs[hh]) * (2 * C * C) + C * C + 256 * t +
                16 * c16 + r4;
      if constexpr (std::is_same<E, BF16>::value) {
        *reinterpret_cast<u32x2*>(pout) = u32x2{cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3])};
      } else {
        *reinterpret_cast<f32x4*>(pout) = v;
      }
    }
  }
  }
  // ---- per-token scalars a, b, c and e^{gamma_last}
  if (wave < HPW && lane < C) {
    float* scal = a.scal + (chunk * a.hv + hs[wave]) * (kScalRows * C);
    const float gm = sm.gam[wave][lane], glast = sm.gam[wave][C - 1];
    const float eg = __expf(gm);
    scal[lane] = eg * sm.rk[lane];
    if constexpr (WQ) scal[C + lane] = eg * sm.rq[lane];
    scal[2 * C + lane] = __expf(glast - gm) * sm.rk[lane];
    scal[3 * C + lane] = lane == 0 ? __expf(glast) : 0.f;
    scal[4 * C + lane] = gm;
    scal[5 * C + lane] = sm.rk[lane];
    scal[7 * C + lane] = eg;
  }
  lds_barrier();  // K and Q are dead: A takes their place
#pragma unroll
  for (int n = 0; n < NTW; n++) {
    const int t = wave + PW * n;
    if (t < NT) {
      int i, j;
      tile_ij(t, i, j);
      const int r = 16 * i + c16, s0 = 16 * j + r4;
      const float fr = sm.rk[r];
      // the four columns' factors as one 16-byte read each, and no branch
      // per element (a masked element may be inf; the select drops it)
      const f32x4 rks = *reinterpret_cast<const f32x4*>(&sm.rk[s0]);
#pragma unroll
      for (int hh = 0; hh < HPW; hh++) {
        const float gr = sm.gam[hh][r], br = sm.bet[hh][r] * fr;
        const f32x4 gs = *reinterpret_cast<const f32x4*>(&sm.gam[hh][s0]);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float val = br * rks[e] * __expf(gr - gs[e]) * rawA[n][e];
          v[e] = s0 + e < r ? val : 0.f;
        }
        *reinterpret_cast<f32x4*>(&sm.u.at[hh][r][s0]) = v;
      }
    }
  }
  lds_barrier();
  // ---- diagonal 16x16 blocks, inverted in registers, written back in place
  for (int blk = wave; blk < HPW * NRT; blk += PW) {
    const int hh = blk / NRT, d = blk % NRT;
    float* A0 = &sm.u.at[hh][16 * d][16 * d];
    const f32x4 inv = inv16(A0, L, lane);
    st_c(A0, L, inv, lane);
  }
  lds_barrier();
  // ---- merge 16 -> 32: [[X, 0], [Y, Z]]^{-1} has lower-left block -Z (Y X)
  if constexpr (C >= 32) {
    for (int m = wave; m < HPW * (NRT / 2); m += PW) {
      const int hh = m / (NRT / 2), b = 32 * (m % (NRT / 2));
      float* at = &sm.u.at[hh][0][0];
      const f32x4 w = mm_tt(ld_ct(at + (b + 16) * L + b, L, lane), ld_c(at + b * L + b, L, lane));
      const f32x4 l = mm_tt(ld_ct(at + (b + 16) * L + b + 16, L, lane), w);
      st_c(at + (b + 16) * L + b, L, -l, lane);
    }
    lds_barrier();
  }
  // ---- merge 32 -> 64: lower-left 32x32 block -Z (Y X), one 16-column
  // strip jc of it per wave; Y is still the original A there
  if constexpr (C == 64) {
    f32x4 l2 = {0.f, 0.f, 0.f, 0.f}, l3 = {0.f, 0.f, 0.f, 0.f};
    const int hh = wave >> 1, jc = wave & 1;
    const bool act = hh < HPW;
    float* at = &sm.u.at[act ? hh : 0][0][0];
    auto blk = [&](int bi, int bj) { return at + 16 * bi * L + 16 * bj; };
    if (act) {
      f32x4 w2, w3;
      if (jc == 0) {  // W_i0 = A_i0 X00 + A_i1 X10
        const f32x4 x00 = ld_c(blk(0, 0), L, lane), x10 = ld_c(blk(1, 0), L, lane);
        w2 = mm_tt(ld_ct(blk(2, 0), L, lane), x00) + mm_tt(ld_ct(blk(2, 1), L, lane), x10);
        w3 = mm_tt(ld_ct(blk(3, 0), L, lane), x00) + mm_tt(ld_ct(blk(3, 1), L, lane), x10);
      } else {        // W_i1 = A_i1 X11
        const f32x4 x11 = ld_c(blk(1, 1), L, lane);
        w2 = mm_tt(ld_ct(blk(2, 1), L, lane), x11);
        w3 = mm_tt(ld_ct(blk(3, 1), L, lane), x11);
      }
      // L_2j = -Z22 W_2j ; L_3j = -(Z32 W_2j + Z33 W_3j)
      l2 = -mm_tt(ld_ct(blk(2, 2), L, lane), w2);
      l3 = -(mm_tt(ld_ct(blk(3, 2), L, lane), w2) + mm_tt(ld_ct(blk(3, 3), L, lane), w3));
    }
    lds_barrier();  // every wave has read the original A blocks
    if (act) {
      st_c(blk(2, jc), L, l2, lane);
      st_c(blk(3, jc), L, l3, lane);
    }
    lds_barrier();
  }
  // ---- Tt = inv diag(beta), upper triangle zero, to the workspace: only its
  // lower 16x16 blocks, packed: block n = i(i+1)/2 + j (row tile i, column
  // tile j <= i) is 256 values, row-major, at 256 n (P the same, C x C
  // further on).  The carries place the blocks in LDS, whose upper blocks
  // stay zero.
  {
#pragma unroll
    for (int hh = 0; hh < HPW; hh++) {
      T* out = reinterpret_cast<T*>(a.tinv) + (chunk * a.hv + hs[hh]) * (2 * C * C);
      for (int idx = tid; idx < NT * 32; idx += PT) {  // 8 values (one 16-byte bf16 word) each
        const int n = idx >> 5, rr = (idx & 31) >> 1, w = idx & 1;
        int i, j;
        tile_ij(n, i, j);
        const int r = 16 * i + rr, s0 = 16 * j + 8 * w;
        float v[8];
#pragma unroll
        for (int h4 = 0; h4 < 2; h4++) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.u.at[hh][r][s0 + 4 * h4]);
          const f32x4 bs = *reinterpret_cast<const f32x4*>(&sm.bet[hh][s0 + 4 * h4]);
#pragma unroll
          for (int e = 0; e < 4; e++) v[4 * h4 + e] = s0 + 4 * h4 + e <= r ? x[e] * bs[e] : 0.f;
        }
        T* dst = out + 256 * n + 16 * rr + 8 * w;
        if constexpr (std::is_same<E, BF16>::value) {
          *reinterpret_cast<u32x4*>(dst) = u32x4{cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3]),
                                                 cvt_bf16x2(v[4], v[5]), cvt_bf16x2(v[6], v[7])};
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
      }
    }
  }
}

// ---------------------------------------------------------------- phase 2
//
// One workgroup per (sequence, v-head, NT*16 columns of d_v), 4*NT waves
// (8 for the split form below).  Waves 4t..4t+3 own column tile t; within it
// wave lw owns token rows 16lw..16lw+15 of the chunk (X, U, O) and d_k rows
// of the state (S).  Per chunk (staged data in LDS buffer b, the next
// chunks' loads in flight):
//   B0 | X = K S -> R, S^T Q^T | B1 | U = Tt R | B2 | O^T = diag(b) S^T Q^T + U^T P^T ;
//        S <- e^{gl} S + K^T diag(c) U ; stage next chunk
// O is formed transposed so each lane owns 4 consecutive columns of one
// token row and writes them with one 8- or 16-byte store.

template <class E, int C, int DK, int NT, bool DB>
struct alignas(16) ScanSmem {
  typedef typename E::store_t T;
  static constexpr int NB = DB ? 2 : 1;            // staging buffers
  static constexpr int PADE = 16 / sizeof(T);
  static constexpr int KLD = DK + PADE;
  // token-indexed arrays along the MFMA K dimension are padded to a whole
  // K step (bf16 chunk 16 -> 32); the padding stays zero
  static constexpr int CW = C > E::KSTEP ? C : E::KSTEP;
  static constexpr int CLD = CW + PADE;
  static constexpr int VLD = C + 4;
  T k[NB][C][KLD];
  T q[NB][C][KLD];
  T tt[NB][C][CLD];
  T p[NB][C][CLD];
  float vt[NB][16 * NT][VLD];  // V^T slice, fp32
  float sc[NB][4][C];          // a, b, c, e^{gamma_last}
  T st[2][NT][16][KLD];        // S^T as operand, double-buffered
  T rt[NT][16][CLD];           // R^T
  T ut[NT][16][CLD];           // U^T
  T u2t[NT][16][CLD];          // (diag(c) U)^T
};

// D += A B where A(16 x K) = M^T for M row-major [K][ld] (fp32 operands,
// K a multiple of 16).  The k of four consecutive steps are regrouped as in
// tile_mma_f32 (step i, lane (r, q): k = kb + 4q + i), so B is one 16-byte
// read per four steps; A is a column of M, four 4-byte reads.
template <int K>
__device__ __forceinline__ f32x4 tile_mma_at_f32(f32x4 acc, const float* M, int ldm, const float* BT, int ldb,
                                                 int lane) {
  static_assert(K % 16 == 0, "K must be a multiple of 16");
  const int r = lane & 15, kq = (lane >> 4) * 4;
#pragma unroll
  for (int kb = 0; kb < K; kb += 16) {
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(BT + r * ldb + kb + kq);
#pragma unroll
    for (int i = 0; i < 4; i++) acc = mfma16(M[(kb + kq + i) * ldm + r], b4[i], acc);
  }
  return acc;
}

// D += A B with A(16 x CW) = K^T rows rb..rb+15, K row-major [C][ldk] bf16:
// each lane gathers its 8 consecutive tokens of one column from LDS.  Tokens
// at or past C (K-step padding) read as zero.
template <int C, int LDK, int CW>
__device__ __forceinline__ f32x4 tile_mma_kt_bf16(f32x4 acc, const uint16_t* K, int rb, const uint16_t* BT, int ldb,
                                                  int lane) {
  const int r = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
  for (int kb = 0; kb < CW; kb += 32) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int s0 = kb + kq + 2 * e;
      const uint32_t lo = (s0 < C) ? K[s0 * LDK + rb + r] : 0u;
      const uint32_t hi = (s0 + 1 < C) ? K[(s0 + 1) * LDK + rb + r] : 0u;
      w[e] = lo | (hi << 16);
    }
    acc = mfma16(__builtin_bit_cast(bf16x8, w), load_frag(BT + r * ldb + kq + kb, BF16()), acc);
  }
  return acc;
}

// D += A B over k < kend (kend a multiple of the MFMA K step, at most KMAX;
// for fp32 a multiple of 16: the steps take the regrouped 16-byte reads of
// tile_mma_f32, all KMAX of them issued first, the products then run for
// the blocks below kend).
template <class E, int KMAX>
__device__ __forceinline__ f32x4 tile_mma_rt(f32x4 acc, const typename E::store_t* A, int lda,
                                             const typename E::store_t* BT, int ldb, int lane, int kend) {
  if constexpr (E::KSTEP == 4 && KMAX % 16 == 0) {
    const int r = lane & 15, kq = (lane >> 4) * 4;
    f32x4 a4[KMAX / 16], b4[KMAX / 16];
#pragma unroll
    for (int j = 0; j < KMAX / 16; j++) {
      a4[j] = *reinterpret_cast<const f32x4*>(A + r * lda + kq + 16 * j);
      b4[j] = *reinterpret_cast<const f32x4*>(BT + r * ldb + kq + 16 * j);
    }
#pragma unroll
    for (int j = 0; j < KMAX / 16; j++) {
      if (16 * j < kend) {
#pragma unroll
        for (int i = 0; i < 4; i++) acc = mfma16(a4[j][i], b4[j][i], acc);
      }
    }
    return acc;
  }
  const int r = lane & 15, kq = (lane >> 4) * E::KPL;
  for (int kb = 0; kb < kend; kb += E::KSTEP)
    acc = mfma16(load_frag(A + r * lda + kq + kb, E()), load_frag(BT + r * ldb + kq + kb, E()), acc);
  return acc;
}

// X = K S and Y = S^T Q^T for one 16-token row tile (fp32 operands, K a
// multiple of 32), with the regrouped reads of tile_mma_f32: the S^T row a
// lane reads is B for X and A for Y, so it is read once for both, and the
// two independent chains interleave.  Reads go in batches of 4 k blocks.
template <int K>
__device__ __forceinline__ void tile_mma_xy_f32(f32x4& X, f32x4& Y, const float* Kr, const float* St,
                                                const float* Qr, int ld, int lane) {
  static_assert(K % 64 == 0 || K == 32, "K");
  constexpr int NB = K >= 64 ? 4 : 2;  // k blocks of 16 per batch
  const int r = lane & 15, kq = (lane >> 4) * 4;
  const float *pk = Kr + r * ld + kq, *ps = St + r * ld + kq, *pq = Qr + r * ld + kq;
#pragma unroll
  for (int kb = 0; kb < K; kb += 16 * NB) {
    f32x4 k4[NB], s4[NB], q4[NB];
#pragma unroll
    for (int j = 0; j < NB; j++) {
      k4[j] = *reinterpret_cast<const f32x4*>(pk + kb + 16 * j);
      s4[j] = *reinterpret_cast<const f32x4*>(ps + kb + 16 * j);
      q4[j] = *reinterpret_cast<const f32x4*>(pq + kb + 16 * j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        X = mfma16(k4[j][i], s4[j][i], X);
        Y = mfma16(s4[j][i], q4[j][i], Y);
      }
  }
}

// Store 4 consecutive values (one lane's accumulator column) contiguously.
__device__ __forceinline__ void st4(uint16_t* p, f32x4 v) {
  u32x2 w = {cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3])};
  *reinterpret_cast<u32x2*>(p) = w;
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }


// SPLIT (one column tile, NT = 1): eight waves, two per SIMD.  Waves 0-3
// carry as above (X, R, U and the state update); waves 4-7 form the output
// (S^T Q^T beside X, then U^T P^T and the o store beside the state update),
// so each phase's products are shared by two waves of a SIMD.
template <class E, int C, int DK, int NT, bool DB, bool SPLIT>
__global__ void __launch_bounds__(256 * NT * (SPLIT ? 2 : 1)) k_scan(ScanArgs a) {
  static_assert(!SPLIT || NT == 1, "the split form has one column tile");
  typedef typename E::store_t T;
  typedef ScanSmem<E, C, DK, NT, DB> SM;
  constexpr int NTH = 256 * NT * (SPLIT ? 2 : 1);  // threads
  constexpr int NRT = C / 16;      // 16-row tiles per chunk
  constexpr int STW = DK / 64;     // state row tiles per wave (per column tile)
  constexpr int KLD = SM::KLD, CLD = SM::CLD;
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int tw = SPLIT ? 0 : wave >> 2, lw = wave & 3;   // column tile, wave within it
  const bool outw = SPLIT && wave >= 4;                 // an output wave of the split form
  const int c16 = lane & 15, r4 = (lane >> 4) * 4;

  // Zero all LDS once: the upper triangles and the K-step padding are read
  // by the matrix cores but never written.
  {
    u32x4* z = reinterpret_cast<u32x4*>(&sm);
    for (int i = tid; i < (int)(sizeof(SM) / 16); i += NTH) z[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // ---- which (sequence, v-head, column block): XCD-aware numbering.  All
  // workgroups reading the same q/k head get the same (id % 8), i.e. the
  // same XCD and L2, since workgroups are dealt round-robin over the 8 XCDs.
  const int nblk = a.dv / (16 * NT);
  const int G = a.hv / a.hk;
  const int GS = G * nblk;                   // workgroups per (seq, qk head)
  const int ngroups = a.num_seqs * a.hk;
  const int xcd = blockIdx.x & 7, m = blockIdx.x >> 3;
  const int grp = (m / GS) * 8 + xcd;
  if (grp >= ngroups) return;
  const int local = m % GS;
  const int hk = grp % a.hk;
  // with variable lengths, sequences in the chunk table's order (longest first)
  const int seq = a.seg_perm ? a.seg_perm[grp / a.hk] : grp / a.hk;
  const int vh = local / nblk;
  const int h = a.tiled ? (hk + vh * a.hk) : (hk * G + vh);
  const int dv0 = (local % nblk) * 16 * NT;

  int s0, s1, cbase;
  if (a.seqlen > 0) {
    s0 = seq * a.seqlen;
    s1 = s0 + a.seqlen;
    cbase = seq * ((a.seqlen + C - 1) / C);
  } else {
    s0 = a.cu_seqlens[seq];
    s1 = a.cu_seqlens[seq + 1];
    cbase = a.chunk_offsets[seq];
  }
  const int nchunks = (s1 - s0 + C - 1) / C;

  lds_barrier();  // zeroing done

  // ---- initial state: wave (tw, lw) owns rows [lw*DK/4, (lw+1)*DK/4) of tile tw
  f32x4 S[STW];
  {
    // the branch encloses the whole loop, so that its loads all issue before
    // the first wait (a branch around each load makes the compiler wait for
    // the loads in flight where it rejoins: one memory round trip each)
    const float* sin = a.state_in ? a.state_in + ((long)seq * a.hv + h) * DK * a.dv : nullptr;
    const int col = dv0 + 16 * tw + c16;
    if (sin) {
#pragma unroll
      for (int t = 0; t < STW; t++)
#pragma unroll
        for (int e = 0; e < 4; e++) S[t][e] = sin[(long)((lw * STW + t) * 16 + r4 + e) * a.dv + col];
    } else {
#pragma unroll
      for (int t = 0; t < STW; t++) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (!outw) {
#pragma unroll
      for (int t = 0; t < STW; t++) st4(&sm.st[0][tw][c16][(lw * STW + t) * 16 + r4], S[t]);
    }
  }

  // ---- staging: a chunk's global loads go into registers ahead of its use
  // (per-thread source offsets are fixed; only a per-chunk base moves), then
  // are written to LDS in the parts its single buffer frees up.
  constexpr int EPV = 16 / sizeof(T);              // elements per 16-byte vector
  constexpr int VPR = DK / EPV;                    // vectors per K/Q row
  constexpr int KQ_V = 2 * C * VPR;                // K and Q vectors per chunk
  constexpr int NKQ = (KQ_V + NTH - 1) / NTH;
  constexpr int NTB = NRT * (NRT + 1) / 2;         // lower 16x16 blocks of Tt (and of P)
  constexpr int BV = 256 / EPV;                    // vectors per block
  constexpr int MH_V = NTB * BV;                   // Tt vectors per chunk (P the same)
  constexpr int M_V = 2 * MH_V;
  constexpr int NM = (M_V + NTH - 1) / NTH;
  constexpr int V_VPR = 16 * NT / EPV;             // V vectors per row
  constexpr int V_V = C * V_VPR;
  constexpr int S_V = C;                           // 4*C scalars = C vectors
  static_assert(V_V <= NTH && S_V <= NTH, "staging");
  const T* qp = reinterpret_cast<const T*>(a.q);
  const T* kp = reinterpret_cast<const T*>(a.k);
  const T* vp = reinterpret_cast<const T*>(a.v);
  const T* mp = reinterpret_cast<const T*>(a.tinv);
  const float* scp = a.scal;
  // Register sets of staged loads: with one LDS buffer, two sets, so that a
  // chunk's loads are issued two chunks ahead of its use (one chunk's
  // compute was too short for them to land).  Set indices are compile-time
  // (the chunk loop runs in pairs), so the sets stay in registers.
  constexpr int PF = DB ? 1 : 2;
  struct Staged {
    u32x4 kq[NKQ], m[NM], v, s;
    int len;  // valid rows of the chunk held
  };
  Staged rs[PF];
  // Each thread's element offsets, computed once: a chunk's load is its base
  // plus the offset, with no 64-bit row-times-stride product per vector.
  // Every load is unconditional (a load inside a branch makes the compiler
  // wait for the loads in flight where the branch rejoins): a row past the
  // sequence's end reads the chunk's first row and is zeroed at the store.
  //
  // K and Q: a thread's vector j is row r0 + RS j of the 2C rows [K; Q], in
  // a fixed column, so the thread keeps one row offset per matrix and the
  // rest of each vector's offset is uniform.
  constexpr int RS = NTH / VPR;                    // rows one vector per thread covers
  constexpr bool ROWSTEP = C % RS == 0;            // else RS is a multiple of C
  static_assert(NTH % VPR == 0 && (ROWSTEP || RS % C == 0), "staging");
  const int r0 = tid / VPR;
  const int kqc = hk * DK + (tid % VPR) * EPV;    // this thread's column
  // matrix (0 K, 1 Q, 2 or more: no vector) and row of vector j
  auto kq_at = [&](int j, int& which, int& r) {
    if constexpr (ROWSTEP) {
      which = RS * j / C;
      r = r0 + (RS * j) % C;
    } else {
      which = (r0 + RS * j) / C;
      r = r0 % C;
    }
  };
  const int rb0 = ROWSTEP ? r0 : r0 % C;
  const long rk0 = (long)rb0 * a.stride_k, rq0 = (long)rb0 * a.stride_q;
  long vo = 0;
  int v0 = 0, vr = C;
  // Tt and P arrive as their lower blocks, packed (block n = i(i+1)/2 + j at
  // 256 n, row-major; P at C x C): each vector's source and its place in the
  // LDS matrix, whose upper blocks keep the zeros written above
  int mo[NM], ml[NM];
#pragma unroll
  for (int j = 0; j < NM; j++) {
    const int idx = min(tid + NTH * j, M_V - 1);
    const int isp = idx >= MH_V, rem = idx - isp * MH_V;
    const int n = rem / BV, w = rem % BV;
    int bi = 0;
    while ((bi + 1) * (bi + 2) / 2 <= n) bi++;
    const int bj = n - bi * (bi + 1) / 2;
    mo[j] = isp * C * C + rem * EPV;
    ml[j] = (16 * bi + w / (16 / EPV)) * CLD + 16 * bj + (w % (16 / EPV)) * EPV;
  }
  if (tid < V_V) {
    const int r = tid / V_VPR, cv = tid % V_VPR;
    vr = r;
    v0 = h * a.dv + dv0 + cv * EPV;
    vo = (long)r * a.stride_v + v0;
  }
  // A chunk's loads by a flat index, in the order the stores below consume
  // them (the load counter retires in order): V (0), Tt and P (1 .. NM), K
  // and Q (NM + 1 .. NM + NKQ), the scalars (NM + NKQ + 1); load_part issues
  // those in [LO, HI).
  constexpr int NLD = NM + NKQ + 2;
  auto load_part = [&](int ch, auto set_, auto lo_, auto hi_) {
    constexpr int LO = decltype(lo_)::value, HI = decltype(hi_)::value;
    Staged& R = rs[decltype(set_)::value];
    const int cs = s0 + ch * C;
    const int clen = min(C, s1 - cs);
    const long blk = (long)(cbase + ch) * a.hv + h;
    if constexpr (LO == 0 && HI > 0) {
      R.len = clen;
      R.v = *reinterpret_cast<const u32x4*>(vp + (long)cs * a.stride_v + (vr < clen ? vo : (long)v0));
    }
    const T* msrc = mp + blk * (2 * C * C);
#pragma unroll
    for (int j = 0; j < NM; j++)
      if (LO <= 1 + j && 1 + j < HI) R.m[j] = *reinterpret_cast<const u32x4*>(msrc + mo[j]);
    const T* kc = kp + (long)cs * a.stride_k;
    const T* qc = qp + (long)cs * a.stride_q;
#pragma unroll
    for (int j = 0; j < NKQ; j++) {
      if (LO <= 1 + NM + j && 1 + NM + j < HI) {
        int which, r;
        kq_at(j, which, r);
        const int dr = ROWSTEP ? (RS * j) % C : 0;  // uniform row step
        const long ro = which == 1 ? rq0 + (long)dr * a.stride_q : rk0 + (long)dr * a.stride_k;
        const T* src = (which == 1 ? qc : kc) + ((which < 2 && r < clen) ? ro : 0) + kqc;
        R.kq[j] = *reinterpret_cast<const u32x4*>(src);
      }
    }
    if constexpr (LO <= NLD - 1 && NLD - 1 < HI)
      R.s = *reinterpret_cast<const u32x4*>(scp + blk * (kScalRows * C) + min(tid, S_V - 1) * 4);
  };
  typedef std::integral_constant<int, 0> LdFirst;
  typedef std::integral_constant<int, NLD> LdAll;
  // With two register sets, the loads two chunks ahead go out in three
  // parts between the phases, none in the first, whose products both waves
  // of each SIMD run (issued there, they held up those products): V, Tt and
  // P after its barrier, K and Q up to LD2 after U's, the last five at the
  // end of the chunk.  (One burst anywhere cost more; the split points were
  // measured on the 8192-token fp32 layer.)
  constexpr int LD1 = 1 + NM;
  constexpr int LD2 = NLD - 5 > LD1 ? NLD - 5 : LD1;
  typedef std::integral_constant<int, LD1> LdSplit1;
  typedef std::integral_constant<int, LD2> LdSplit2;

  // The next chunk's staging goes in three parts, each as soon as no wave
  // reads that array of the current chunk any more (in a single buffer):
  // V^T once every wave is past R (after B1), Tt once every wave is past U
  // (after B2), and the rest at the end of the chunk.
  auto store_v = [&](int b, auto set_) {
    Staged& R = rs[decltype(set_)::value];
    if (R.len < C) {
      // the sequence's last, partial chunk: rows past its end are zero (a
      // branch with no memory access, taken by every lane or none)
#pragma unroll
      for (int j = 0; j < NKQ; j++) {
        int which, r;
        kq_at(j, which, r);
        if (r >= R.len) R.kq[j] = u32x4{0u, 0u, 0u, 0u};
      }
      if (vr >= R.len) R.v = u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < V_V) {
      const int r = tid / V_VPR, cv = tid % V_VPR;
      const T* e = reinterpret_cast<const T*>(&R.v);
#pragma unroll
      for (int i = 0; i < EPV; i++) sm.vt[b][cv * EPV + i][r] = E::to_f32(e[i]);
    }
  };
  auto store_tt = [&](int b, auto set_) {
    const Staged& R = rs[decltype(set_)::value];
#pragma unroll
    for (int j = 0; j < NM; j++)
      if (tid + NTH * j < MH_V) *reinterpret_cast<u32x4*>(&sm.tt[b][0][0] + ml[j]) = R.m[j];
  };
  auto store_rest = [&](int b, auto set_) {
    const Staged& R = rs[decltype(set_)::value];
    const int cve = (tid % VPR) * EPV;
#pragma unroll
    for (int j = 0; j < NKQ; j++) {
      int which, r;
      kq_at(j, which, r);
      if (which < 2) *reinterpret_cast<u32x4*>(which ? &sm.q[b][r][cve] : &sm.k[b][r][cve]) = R.kq[j];
    }
#pragma unroll
    for (int j = 0; j < NM; j++) {
      const int idx = tid + NTH * j;
      if (idx >= MH_V && idx < M_V) *reinterpret_cast<u32x4*>(&sm.p[b][0][0] + ml[j]) = R.m[j];
    }
    if (tid < S_V) *reinterpret_cast<u32x4*>(&sm.sc[b][0][0] + tid * 4) = R.s;
  };

  typedef std::integral_constant<int, 0> Set0;
  typedef std::integral_constant<int, PF - 1> Set1;  // the second set (the first when PF = 1)
  if (nchunks > 0) {
    load_part(0, Set0(), LdFirst(), LdAll());
    if (PF == 2) load_part(min(1, nchunks - 1), Set1(), LdFirst(), LdAll());
    store_v(0, Set0());
    store_tt(0, Set0());
    store_rest(0, Set0());
  }
  T* obase = reinterpret_cast<T*>(a.o) + (long)h * a.dv + dv0 + 16 * tw + r4;
  // One chunk; with PF = 2, chunk ch's loads went to set ch % 2 and its
  // chunk + 2 loads go there again once it is stored (at the end of chunk
  // ch - 1), chunk ch + 1 is stored from the other set.
  auto chunk_step = [&](int ch, auto par_) {
    constexpr int P = decltype(par_)::value;
    typedef std::integral_constant<int, PF == 2 ? P : 0> LoadSet;
    typedef std::integral_constant<int, PF == 2 ? 1 - P : 0> StoreSet;
    const int b = DB ? (ch & 1) : 0;
    const int nb = DB ? (b ^ 1) : 0;
    const int sb = ch & 1;                 // state operand buffer read this chunk
    const int cs = s0 + ch * C;
    const int clen = min(C, s1 - cs);
    lds_barrier();                       // B0: staged chunk and S^T visible
    // one register set: the next chunk's loads go out first, as it is stored
    // during this chunk (unconditional, for the reason given below)
    if constexpr (PF == 1) load_part(min(ch + 1, nchunks - 1), LoadSet(), LdFirst(), LdAll());

    // ---- X = K S, R = V - diag(a) X -> R^T; and Y = S^T Q^T for the
    // output, which needs only the chunk's start state
    f32x4 Y = {0.f, 0.f, 0.f, 0.f};
    if (lw < NRT) {
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      if constexpr (SPLIT) {
        if (!outw) X = tile_mma<E, DK, true>(X, &sm.k[b][16 * lw][0], KLD, &sm.st[sb][tw][0][0], KLD, lane);
        else Y = tile_mma<E, DK, true>(Y, &sm.st[sb][tw][0][0], KLD, &sm.q[b][16 * lw][0], KLD, lane);
      } else if constexpr (E::KSTEP == 4) {
        tile_mma_xy_f32<DK>(X, Y, reinterpret_cast<const float*>(&sm.k[b][16 * lw][0]),
                            reinterpret_cast<const float*>(&sm.st[sb][tw][0][0]),
                            reinterpret_cast<const float*>(&sm.q[b][16 * lw][0]), KLD, lane);
      } else {
        X = tile_mma<E, DK, true>(X, &sm.k[b][16 * lw][0], KLD, &sm.st[sb][tw][0][0], KLD, lane);
        Y = tile_mma<E, DK, true>(Y, &sm.st[sb][tw][0][0], KLD, &sm.q[b][16 * lw][0], KLD, lane);
      }
      const int s = 16 * lw + r4;
      if (!outw) st4(&sm.rt[tw][c16][s], ld4(&sm.vt[b][16 * tw + c16][s]) - ld4(&sm.sc[b][0][s]) * X);
    }
    lds_barrier();                       // B1
    // Two register sets: the first part of the loads two chunks ahead.
    // Unconditional: past the last chunk they load the last one again, into
    // a set that is never stored.  (Under a branch the compiler would count
    // them as maybe not issued and wait for the newest of them where the
    // older set is stored.)
    const int lch = min(ch + 2, nchunks - 1);
    if constexpr (PF == 2) load_part(lch, LoadSet(), LdFirst(), LdSplit1());
    store_v(nb, StoreSet());    // every wave is past this chunk's V^T
    // ---- U = Tt R (Tt lower triangular: k < 16(lw+1)) -> U^T, (diag(c) U)^T
    if (lw < NRT && !outw) {
      const int kend = ((16 * (lw + 1) + E::KSTEP - 1) / E::KSTEP) * E::KSTEP;
      f32x4 U = {0.f, 0.f, 0.f, 0.f};
      U = tile_mma_rt<E, C>(U, &sm.tt[b][16 * lw][0], CLD, &sm.rt[tw][0][0], CLD, lane, kend);
      const int s = 16 * lw + r4;
      st4(&sm.ut[tw][c16][s], U);
      st4(&sm.u2t[tw][c16][s], ld4(&sm.sc[b][2][s]) * U);
    }
    lds_barrier();                       // B2
    if constexpr (PF == 2) load_part(lch, LoadSet(), LdSplit1(), LdSplit2());
    store_tt(nb, StoreSet());   // every wave is past this chunk's Tt
    // ---- O^T = diag(b) (S^T Q^T) + U^T P^T, tokens 16lw..16lw+15
    if (lw < NRT && (!SPLIT || outw)) {
      const int kend = ((16 * (lw + 1) + E::KSTEP - 1) / E::KSTEP) * E::KSTEP;
      f32x4 PU = {0.f, 0.f, 0.f, 0.f};
      PU = tile_mma_rt<E, C>(PU, &sm.ut[tw][0][0], CLD, &sm.p[b][16 * lw][0], CLD, lane, kend);
      const int r = 16 * lw + c16;
      if (r < clen) st4(obase + (long)(cs + r) * a.hv * a.dv, sm.sc[b][1][r] * Y + PU);
    }
    // ---- S <- e^{gamma_last} S + K^T diag(c) U  -> S^T operand for the next chunk
    if (!outw) {
      const float gl = sm.sc[b][3][0];
#pragma unroll
      for (int t = 0; t < STW; t++) {
        const int rb = (lw * STW + t) * 16;
        f32x4 acc = S[t] * gl;
        if constexpr (std::is_same<E, BF16>::value) {
          acc = tile_mma_kt_bf16<C, KLD, SM::CW>(acc, &sm.k[b][0][0], rb, &sm.u2t[tw][0][0], CLD, lane);
        } else {
          acc = tile_mma_at_f32<C>(acc, reinterpret_cast<const float*>(&sm.k[b][0][rb]), KLD,
                                   reinterpret_cast<const float*>(&sm.u2t[tw][0][0]), CLD, lane);
        }
        S[t] = acc;
        st4(&sm.st[sb ^ 1][tw][c16][rb + r4], acc);
      }
    }
    // ---- stage the next chunk (single-buffered: wait until all waves are
    // done with this chunk's staged data).  Like the loads, the stores have
    // no branch around them: after the last chunk they write the last chunk
    // again, which nothing reads.
    if constexpr (PF == 2) load_part(lch, LoadSet(), LdSplit2(), LdAll());
    if (!DB) lds_barrier();
    store_rest(nb, StoreSet());
  };
  // in pairs (the register sets are compile-time); an odd last chunk leaves
  // the loop between the two steps
  for (int ch = 0; ch < nchunks; ch += 2) {
    chunk_step(ch, std::integral_constant<int, 0>());
    if (ch + 1 >= nchunks) break;
    chunk_step(ch + 1, std::integral_constant<int, 1>());
  }

  // ---- final state
  if (a.state_out && !outw) {
    float* so = a.state_out + ((long)seq * a.hv + h) * DK * a.dv;
    const int col = dv0 + 16 * tw + c16;
#pragma unroll
    for (int t = 0; t < STW; t++) {
      const int rb = (lw * STW + t) * 16;
#pragma unroll
      for (int e = 0; e < 4; e++) so[(long)(rb + r4 + e) * a.dv + col] = S[t][e];
    }
  }
}

template <class E, int C, int DK>
hipError_t launch_prepare_t(const ScanArgs& a, hipStream_t s) {
  const int G = a.hv / a.hk;
  const dim3 block(64 * kPrepWaves);
  const int hpw = G % 2 == 0 ? 2 : 1;
  const dim3 grid((unsigned)((long)a.max_chunks * (a.hv / hpw)));  // one (chunk, head group) per workgroup
  if (seg_path(a)) {
    if (hpw == 2) hipLaunchKernelGGL((k_prepare<E, C, DK, 2, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_prepare<E, C, DK, 1, false>), grid, block, 0, s, a);
  } else {
    if (hpw == 2) hipLaunchKernelGGL((k_prepare<E, C, DK, 2, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_prepare<E, C, DK, 1, true>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <class E, int C, int DK>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  constexpr bool BF = std::is_same<E, BF16>::value;
  // Sequential carry for what the segment-parallel path does not take:
  // bf16 chunk 16 with two 16-column tiles per workgroup (8 waves), LDS
  // double-buffered; fp32 with one tile (8 waves, the split form),
  // single-buffered (the fp32 tiles fill the LDS)
  constexpr int NT = BF ? 2 : 1;
  constexpr bool SPLIT = !BF;  // fp32: eight waves per tile, the output formed by waves of its own
  const int GS = (a.hv / a.hk) * (a.dv / (16 * NT));
  const int ngroups = a.num_seqs * a.hk;
  const int per_xcd = (ngroups + 7) / 8;
  dim3 grid(8 * per_xcd * GS), block(256 * NT * (SPLIT ? 2 : 1));
  hipLaunchKernelGGL((k_scan<E, C, DK, NT, BF, SPLIT>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <class E>
hipError_t dispatch_prepare(const ScanArgs& a, hipStream_t s) {
  if (a.dk == 128) {
    if (a.chunk == 64) return launch_prepare_t<E, 64, 128>(a, s);
    if (a.chunk == 32) return launch_prepare_t<E, 32, 128>(a, s);
    if (a.chunk == 16) return launch_prepare_t<E, 16, 128>(a, s);
  } else if (a.dk == 64) {
    if (a.chunk == 64) return launch_prepare_t<E, 64, 64>(a, s);
    if (a.chunk == 32) return launch_prepare_t<E, 32, 64>(a, s);
    if (a.chunk == 16) return launch_prepare_t<E, 16, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class E>
hipError_t dispatch_scan(const ScanArgs& a, hipStream_t s) {
  if (a.dk == 128) {
    if (a.chunk == 64) return launch_scan_t<E, 64, 128>(a, s);
    if (a.chunk == 32) return launch_scan_t<E, 32, 128>(a, s);
    if (a.chunk == 16) return launch_scan_t<E, 16, 128>(a, s);
  } else if (a.dk == 64) {
    if (a.chunk == 64) return launch_scan_t<E, 64, 64>(a, s);
    if (a.chunk == 32) return launch_scan_t<E, 32, 64>(a, s);
    if (a.chunk == 16) return launch_scan_t<E, 16, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_table(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prepare(const ScanArgs& a, hipStream_t s) {
  if (a.max_chunks == 0) return hipSuccess;
  return a.dtype == 1 ? dispatch_prepare<BF16>(a, s) : dispatch_prepare<F32>(a, s);
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  if (seg_path(a)) return launch_seg(a, s);
  return a.dtype == 1 ? dispatch_scan<BF16>(a, s) : dispatch_scan<F32>(a, s);
}

}  // namespace gdn
