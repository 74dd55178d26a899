// prefill.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The oxydllm 0.0.0-alpha.12.2 release notes ("New Features", Gated DeltaNet
// runtime; "Performance", Gated DeltaNet fast paths) run prefill as a chunked
// parallel scan: the state-independent work of every chunk is done in batch,
// then a sequential loop carries the state across chunks.  For a chunk of C
// tokens (gamma_r = g_0 + ... + g_r inside the chunk, k_hat = rk k, q_hat = rq q):
//
//   A[r,s] = beta_r e^{gamma_r - gamma_s} k_hat_r . k_hat_s     (s < r)
//   Tt     = (I + A)^{-1} diag(beta)
//   U      = Tt (V - diag(e^gamma) K_hat S)                 -- new values
//   P[r,s] = e^{gamma_r - gamma_s} q_hat_r . k_hat_s          (s <= r)
//   O      = diag(e^gamma) Q_hat S + P U
//   S     <- e^{gamma_last} S + K_hat^T diag(e^{gamma_last - gamma}) U
//
// Phase 1 (k_prepare): one workgroup per (chunk, v-head) builds A from
// K K^T on the matrix cores and inverts I + A blockwise -- the doubling
// product (I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8) on each 16x16 diagonal
// block (N^16 = 0), then pairwise merging 16 -> 32 -> 64 with
// [[X,0],[Y,Z]]^{-1} = [[X^-1,0],[-Z^-1 Y X^-1, Z^-1]] -- never powers of the
// whole 64x64 block, which overflow fp32 on repeated tokens (the notes'
// failure of plain doubling at chunk 64).  It writes Tt to the workspace.
//
// Phase 2 (k_scan): one workgroup per (sequence, v-head, 16 columns of d_v)
// walks the chunks in order with its 128x16 fp32 slice of S in registers.
// Each chunk it stages K, Q, V and Tt in LDS, forms P on the matrix cores
// (state independent, so it overlaps the dependent chain), then runs the
// chain X = K S -> U -> (O, S).  Only Tt crosses HBM between the phases;
// P, U and the per-chunk states never leave the chip.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr float kL2Eps = 1e-6f;

// ------------------------------------------------------------ chunk table
// chunk_offsets[i] = sum_{j<i} ceil(len_j / C).  One workgroup; sequential
// over blocks of 1024 sequences, scan inside a block.
__global__ void __launch_bounds__(1024) k_chunk_table(ScanArgs a) {
  __shared__ int carry;
  __shared__ int buf[1024];
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < a.num_seqs; base += 1024) {
    const int i = base + threadIdx.x;
    int n = 0;
    if (i < a.num_seqs) {
      const int len = a.cu_seqlens[i + 1] - a.cu_seqlens[i];
      n = (len + a.chunk - 1) / a.chunk;
    }
    buf[threadIdx.x] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
      int v = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += v;
      __syncthreads();
    }
    if (i < a.num_seqs) a.chunk_offsets[i + 1] = carry + buf[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 1023) carry += buf[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.chunk_offsets[0] = 0;
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

template <class E, int C, int DK>
struct alignas(16) PrepSmem {
  typedef typename E::store_t T;
  static constexpr int KLD = DK + 16 / sizeof(T);  // row pad: 16 bytes
  static constexpr int ALD = C + 1;
  static constexpr int SLD = 17;
  T k[C][KLD];
  float at[C][ALD];            // A, then (I + A)^{-1} in place
  float sc[4][4][16][SLD];     // per-wave 16x16 scratch
  float w1[32][33];
  float gam[C], bet[C], rk[C];
};

template <class E, int C, int DK>
__global__ void __launch_bounds__(256) k_prepare(ScanArgs a) {
  typedef typename E::store_t T;
  typedef PrepSmem<E, C, DK> SM;
  __shared__ SM sm;
  const int h = blockIdx.y;
  int seq, start, len;
  if (!chunk_of(a, C, blockIdx.x, seq, start, len)) return;
  const int hk = a.tiled ? (h % a.hk) : (h / (a.hv / a.hk));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- stage K rows (zero past the end of the sequence), g, beta
  {
    constexpr int VPR = DK * sizeof(T) / 16;  // 16-byte vectors per row
    const T* kp = reinterpret_cast<const T*>(a.k);
    for (int idx = tid; idx < C * VPR; idx += 256) {
      const int r = idx / VPR, cv = idx % VPR;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (r < len)
        w = *reinterpret_cast<const u32x4*>(kp + (long)(start + r) * a.stride_k + (long)hk * DK + cv * (16 / sizeof(T)));
      *reinterpret_cast<u32x4*>(&sm.k[r][cv * (16 / sizeof(T))]) = w;
    }
  }
  if (wave == 0) {
    float gv = 0.f, bv = 0.f;
    if (lane < len) {
      gv = a.g[(long)(start + lane) * a.hv + h];
      bv = a.beta[(long)(start + lane) * a.hv + h];
    }
    const float gm = wave_prefix_sum(gv, lane);
    if (lane < C) {
      sm.gam[lane] = gm;
      sm.bet[lane] = bv;
    }
  }
  __syncthreads();
  // ---- row norms of K
  {
    constexpr int TPR = 256 / C;  // threads per row
    constexpr int EPT = DK / TPR;
    const int r = tid / TPR, part = tid % TPR;
    float ss = 0.f;
#pragma unroll 8
    for (int i = 0; i < EPT; i++) {
      const float x = E::to_f32(sm.k[r][part * EPT + i]);
      ss += x * x;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
    if (part == 0) sm.rk[r] = a.l2norm ? 1.0f / sqrtf(ss + kL2Eps) : 1.0f;
  }
  __syncthreads();
  // ---- A = strict lower part of diag(beta) (decay * K_hat K_hat^T)
  {
    constexpr int NT = C / 16;
    for (int t = wave; t < NT * NT; t += 4) {
      const int i = t / NT, j = t % NT;
      const int c = lane & 15, r0 = (lane >> 4) * 4;
      if (j > i) {
#pragma unroll
        for (int e = 0; e < 4; e++) sm.at[16 * i + r0 + e][16 * j + c] = 0.f;
        continue;
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = tile_mma<E, DK>(acc, &sm.k[16 * i][0], SM::KLD, &sm.k[16 * j][0], SM::KLD, lane);
      const int s = 16 * j + c;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int r = 16 * i + r0 + e;
        float v = 0.f;
        if (s < r) v = sm.bet[r] * sm.rk[r] * sm.rk[s] * __expf(sm.gam[r] - sm.gam[s]) * acc[e];
        sm.at[r][s] = v;
      }
    }
  }
  __syncthreads();
  // ---- 16x16 diagonal blocks: (I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8)
  if (wave < C / 16) {
    float* N = &sm.at[16 * wave][16 * wave];
    float* s0 = &sm.sc[wave][0][0][0];
    float* s1 = &sm.sc[wave][1][0][0];
    float* s2 = &sm.sc[wave][2][0][0];
    float* s3 = &sm.sc[wave][3][0][0];
    constexpr int L = SM::ALD, S = SM::SLD;
    f32x4 n2 = mm16_f32<16>(N, L, N, L, lane);
    st16(s0, S, n2, lane);
    wave_lds_sync();
    f32x4 n4 = mm16_f32<16>(s0, S, s0, S, lane);
    st16(s1, S, n4, lane);
    wave_lds_sync();
    f32x4 n8 = mm16_f32<16>(s1, S, s1, S, lane);
    st16_plus_i(s2, S, n8, lane);  // I + N^8
    st16_plus_i(s0, S, n2, lane);  // I + N^2
    st16_plus_i(s1, S, n4, lane);  // I + N^4
    {  // I - N
      const int c = lane & 15, r0 = (lane >> 4) * 4;
#pragma unroll
      for (int e = 0; e < 4; e++) s3[(r0 + e) * S + c] = (r0 + e == c ? 1.f : 0.f) - N[(r0 + e) * L + c];
    }
    wave_lds_sync();
    f32x4 p = mm16_f32<16>(s3, S, s0, S, lane);
    wave_lds_sync();
    st16(s3, S, p, lane);
    wave_lds_sync();
    p = mm16_f32<16>(s3, S, s1, S, lane);
    wave_lds_sync();
    st16(s3, S, p, lane);
    wave_lds_sync();
    p = mm16_f32<16>(s3, S, s2, S, lane);
    st16(N, L, p, lane);
  }
  __syncthreads();
  // ---- merge 16 -> 32: lower-left block L = -Z (Y X)
  if (C >= 32 && wave < C / 32) {
    const int b = 32 * wave;
    constexpr int L = SM::ALD, S = SM::SLD;
    float* X = &sm.at[b][b];
    float* Z = &sm.at[b + 16][b + 16];
    float* Y = &sm.at[b + 16][b];
    float* s0 = &sm.sc[wave][0][0][0];
    f32x4 w = mm16_f32<16>(Y, L, X, L, lane);
    st16(s0, S, w, lane);
    wave_lds_sync();
    f32x4 l = mm16_f32<16>(Z, L, s0, S, lane);
    st16(Y, L, -l, lane);
  }
  __syncthreads();
  // ---- merge 32 -> 64
  if (C == 64) {
    constexpr int L = SM::ALD;
    const int i = wave >> 1, j = wave & 1;  // 16x16 tile of the 32x32 block
    // W1 = Y X with Y = A[32:64, 0:32], X = inv[0:32, 0:32] (lower: k >= j)
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    for (int kb = j; kb < 2; kb++) {
      f32x4 t = mm16_f32<16>(&sm.at[32 + 16 * i][16 * kb], L, &sm.at[16 * kb][16 * j], L, lane);
      w += t;
    }
    st16(&sm.w1[16 * i][16 * j], 33, w, lane);
    __syncthreads();
    // L = -Z W1 with Z = inv[32:64, 32:64] (lower: k <= i)
    f32x4 l = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb <= i; kb++) {
      f32x4 t = mm16_f32<16>(&sm.at[32 + 16 * i][32 + 16 * kb], L, &sm.w1[16 * kb][16 * j], 33, lane);
      l += t;
    }
    st16(&sm.at[32 + 16 * i][16 * j], L, -l, lane);
  }
  __syncthreads();
  // ---- Tt = inv diag(beta), upper triangle zero, to the workspace
  {
    T* out = reinterpret_cast<T*>(a.tinv) + ((long)blockIdx.x * a.hv + h) * (C * C);
    for (int idx = tid; idx < C * C; idx += 256) {
      const int r = idx / C, s = idx % C;
      const float v = s <= r ? sm.at[r][s] * sm.bet[s] : 0.f;
      out[idx] = E::from_f32(v);
    }
  }
}

// ---------------------------------------------------------------- phase 2

template <class E, int C, int DK>
struct alignas(16) ScanSmem {
  typedef typename E::store_t T;
  static constexpr bool KT = std::is_same<E, BF16>::value;  // keep K^T for the S update
  static constexpr int PADE = 16 / sizeof(T);
  static constexpr int KLD = DK + PADE;
  // arrays indexed by token along the MFMA K dimension are padded to a whole
  // K step (bf16 chunk 16 -> 32 columns); the padding stays zero
  static constexpr int CW = C > E::KSTEP ? C : E::KSTEP;
  static constexpr int CLD = CW + PADE;
  T k[C][KLD];
  T kt[KT ? DK : 1][CLD];
  T q[C][KLD];
  T tt[C][CLD];
  T p[C][CLD];
  T st[16][KLD];     // S^T (16 columns of d_v x d_k) as operand
  T rt[16][CLD];     // R^T
  T ut[16][CLD];     // U^T
  T u2t[16][CLD];    // (diag(e^{gl - gamma} rk) U)^T
  float v[C][16];
  float rk[C], rq[C], gam[C], eg[C], egc[C];
  float gl;
};

// D += A B where A(16 x K) = M^T for M row-major [K][ld] (fp32 operands).
template <int K>
__device__ __forceinline__ f32x4 tile_mma_at_f32(f32x4 acc, const float* M, int ldm, const float* BT, int ldb,
                                                 int lane) {
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < K; kb += 4) acc = mfma16(M[(kb + q) * ldm + r], BT[r * ldb + kb + q], acc);
  return acc;
}

template <class E>
__device__ __forceinline__ f32x4 tile_mma_rt(f32x4 acc, const typename E::store_t* A, int lda,
                                             const typename E::store_t* BT, int ldb, int lane, int kend) {
  const int r = lane & 15, kq = (lane >> 4) * E::KPL;
  for (int kb = 0; kb < kend; kb += E::KSTEP)
    acc = mfma16(load_frag(A + r * lda + kq + kb, E()), load_frag(BT + r * ldb + kq + kb, E()), acc);
  return acc;
}

// Write 4 consecutive values of one column into a transposed [16][ld] array.
__device__ __forceinline__ void st_col4(uint16_t* p, f32x4 v) {
  u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *reinterpret_cast<u32x2*>(p) = w;
}
__device__ __forceinline__ void st_col4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

template <class E, int C, int DK>
__global__ void __launch_bounds__(256) k_scan(ScanArgs a) {
  typedef typename E::store_t T;
  typedef ScanSmem<E, C, DK> SM;
  constexpr int NRT = C / 16;      // 16-row tiles per chunk
  constexpr int STW = DK / 64;     // S tiles (16 rows) per wave
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Zero all staging memory once: the upper triangle of P and the K-step
  // padding are read by the matrix cores but never written.
  {
    u32x4* z = reinterpret_cast<u32x4*>(&sm);
    for (int i = tid; i < (int)(sizeof(SM) / 16); i += 256) z[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }

  // ---- which (sequence, v-head, column tile): XCD-aware numbering.  All
  // workgroups reading the same q/k head get the same (id % 8), i.e. the
  // same XCD and L2, since workgroups are dealt round-robin over the 8 XCDs.
  const int ntiles = a.dv / 16;
  const int G = a.hv / a.hk;
  const int GS = G * ntiles;                 // workgroups per (seq, qk head)
  const int ngroups = a.num_seqs * a.hk;
  const int xcd = blockIdx.x & 7, m = blockIdx.x >> 3;
  const int grp = (m / GS) * 8 + xcd;
  if (grp >= ngroups) return;
  const int local = m % GS;
  const int seq = grp / a.hk, hk = grp % a.hk;
  const int vh = local / ntiles;             // which of the G v-heads
  const int h = a.tiled ? (hk + vh * a.hk) : (hk * G + vh);
  const int dv0 = (local % ntiles) * 16;

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

  // ---- initial state slice: wave w owns rows [w*DK/4, (w+1)*DK/4)
  f32x4 S[STW];
  {
    const int c = lane & 15, r0 = (lane >> 4) * 4;
    const float* sin = a.state_in ? a.state_in + ((long)seq * a.hv + h) * DK * a.dv : nullptr;
#pragma unroll
    for (int t = 0; t < STW; t++) {
      const int rb = (wave * STW + t) * 16;
#pragma unroll
      for (int e = 0; e < 4; e++) S[t][e] = sin ? sin[(long)(rb + r0 + e) * a.dv + dv0 + c] : 0.f;
      st_col4(&sm.st[c][rb + r0], S[t]);
    }
  }

  const T* qp = reinterpret_cast<const T*>(a.q);
  const T* kp = reinterpret_cast<const T*>(a.k);
  const T* vp = reinterpret_cast<const T*>(a.v);
  T* op = reinterpret_cast<T*>(a.o);
  const T* tp = reinterpret_cast<const T*>(a.tinv);

  for (int ch = 0; ch < nchunks; ch++) {
    const int cs = s0 + ch * C;
    const int clen = min(C, s1 - cs);
    __syncthreads();  // previous chunk finished with the staging buffers
    // ---- stage K, Q (+K^T), V slice, Tt; zero rows past the end
    {
      constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
      constexpr int VPR = DK / EPV;
      for (int idx = tid; idx < 2 * C * VPR; idx += 256) {
        const int which = idx / (C * VPR);  // 0: K, 1: Q
        const int rem = idx % (C * VPR);
        const int r = rem / VPR, cv = rem % VPR;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (r < clen) {
          const T* src = which ? qp + (long)(cs + r) * a.stride_q : kp + (long)(cs + r) * a.stride_k;
          w = *reinterpret_cast<const u32x4*>(src + (long)hk * DK + cv * EPV);
        }
        T* dst = which ? &sm.q[r][cv * EPV] : &sm.k[r][cv * EPV];
        *reinterpret_cast<u32x4*>(dst) = w;
        if (SM::KT && which == 0) {
          const T* e8 = reinterpret_cast<const T*>(&w);
#pragma unroll
          for (int e = 0; e < EPV; e++) sm.kt[SM::KT ? cv * EPV + e : 0][r] = e8[e];
        }
      }
      // Tt: C x C
      const T* tsrc = tp + ((long)(cbase + ch) * a.hv + h) * (C * C);
      for (int idx = tid; idx < C * C / EPV; idx += 256) {
        const int r = idx / (C / EPV), cv = idx % (C / EPV);
        *reinterpret_cast<u32x4*>(&sm.tt[r][cv * EPV]) = *reinterpret_cast<const u32x4*>(tsrc + idx * EPV);
      }
      // V slice: C x 16
      for (int idx = tid; idx < C * 16; idx += 256) {
        const int r = idx / 16, c = idx % 16;
        sm.v[r][c] = r < clen ? E::to_f32(vp[(long)(cs + r) * a.stride_v + (long)h * a.dv + dv0 + c]) : 0.f;
      }
      if (wave == 0) {
        const float gv = lane < clen ? a.g[(long)(cs + lane) * a.hv + h] : 0.f;
        const float gm = wave_prefix_sum(gv, lane);
        const float glast = __shfl(gm, C - 1, 64);
        if (lane < C) {
          sm.gam[lane] = gm;
          sm.eg[lane] = __expf(gm);
          sm.egc[lane] = __expf(glast - gm);
        }
        if (lane == 0) sm.gl = __expf(glast);
      }
    }
    __syncthreads();
    // ---- row norms of K and Q
    {
      constexpr int TPR = 128 / C;
      constexpr int EPT = DK / TPR;
      const int which = tid >> 7;  // 0: K, 1: Q
      const int r = (tid & 127) / TPR, part = (tid & 127) % TPR;
      const T* row = which ? &sm.q[r][part * EPT] : &sm.k[r][part * EPT];
      float ss = 0.f;
#pragma unroll 8
      for (int i = 0; i < EPT; i++) {
        const float x = E::to_f32(row[i]);
        ss += x * x;
      }
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
      if (part == 0) {
        const float inv = a.l2norm ? 1.0f / sqrtf(ss + kL2Eps) : 1.0f;
        if (which) sm.rq[r] = a.scale * inv; else sm.rk[r] = inv;
      }
    }
    __syncthreads();
    // ---- P (state independent) and X = K S, Y = Q S
    {
      const int c = lane & 15, r0 = (lane >> 4) * 4;
      for (int t = wave; t < NRT * (NRT + 1) / 2; t += 4) {
        int i = 0, rem = t;  // t -> (i, j), j <= i
        while (rem > i) { rem -= i + 1; i++; }
        const int j = rem;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = tile_mma<E, DK>(acc, &sm.q[16 * i][0], SM::KLD, &sm.k[16 * j][0], SM::KLD, lane);
        const int s = 16 * j + c;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int r = 16 * i + r0 + e;
          const float v = s <= r ? __expf(sm.gam[r] - sm.gam[s]) * sm.rq[r] * sm.rk[s] * acc[e] : 0.f;
          sm.p[r][s] = E::from_f32(v);
        }
      }
    }
    f32x4 Y = {0.f, 0.f, 0.f, 0.f};
    if (wave < NRT) {
      const int i = wave;
      const int c = lane & 15, r0 = (lane >> 4) * 4;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      X = tile_mma<E, DK>(X, &sm.k[16 * i][0], SM::KLD, &sm.st[0][0], SM::KLD, lane);
      Y = tile_mma<E, DK>(Y, &sm.q[16 * i][0], SM::KLD, &sm.st[0][0], SM::KLD, lane);
      f32x4 R;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int r = 16 * i + r0 + e;
        R[e] = sm.v[r][c] - sm.eg[r] * sm.rk[r] * X[e];
      }
      st_col4(&sm.rt[c][16 * i + r0], R);
    }
    __syncthreads();
    // ---- U = Tt R (Tt lower triangular: k < 16(i+1))
    f32x4 U = {0.f, 0.f, 0.f, 0.f};
    if (wave < NRT) {
      const int i = wave;
      const int c = lane & 15, r0 = (lane >> 4) * 4;
      const int kend = ((16 * (i + 1) + E::KSTEP - 1) / E::KSTEP) * E::KSTEP;
      U = tile_mma_rt<E>(U, &sm.tt[16 * i][0], SM::CLD, &sm.rt[0][0], SM::CLD, lane, kend);
      f32x4 U2;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int r = 16 * i + r0 + e;
        U2[e] = sm.egc[r] * sm.rk[r] * U[e];
      }
      st_col4(&sm.ut[c][16 * i + r0], U);
      st_col4(&sm.u2t[c][16 * i + r0], U2);
    }
    __syncthreads();
    // ---- O = diag(e^gamma rq) Y + P U
    if (wave < NRT) {
      const int i = wave;
      const int c = lane & 15, r0 = (lane >> 4) * 4;
      const int kend = ((16 * (i + 1) + E::KSTEP - 1) / E::KSTEP) * E::KSTEP;
      f32x4 PU = {0.f, 0.f, 0.f, 0.f};
      PU = tile_mma_rt<E>(PU, &sm.p[16 * i][0], SM::CLD, &sm.ut[0][0], SM::CLD, lane, kend);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int r = 16 * i + r0 + e;
        if (r < clen) {
          const float ov = sm.eg[r] * sm.rq[r] * Y[e] + PU[e];
          op[((long)(cs + r) * a.hv + h) * a.dv + dv0 + c] = E::from_f32(ov);
        }
      }
    }
    // ---- S <- e^{gamma_last} S + K^T U2
    {
      const int c = lane & 15, r0 = (lane >> 4) * 4;
      const float gl = sm.gl;
#pragma unroll
      for (int t = 0; t < STW; t++) {
        const int rb = (wave * STW + t) * 16;
        f32x4 acc = S[t] * gl;
        if constexpr (SM::KT) {
          acc = tile_mma<E, C>(acc, &sm.kt[SM::KT ? rb : 0][0], SM::CLD, &sm.u2t[0][0], SM::CLD, lane);
        } else {
          acc = tile_mma_at_f32<C>(acc, reinterpret_cast<const float*>(&sm.k[0][rb]), SM::KLD,
                                   reinterpret_cast<const float*>(&sm.u2t[0][0]), SM::CLD, lane);
        }
        S[t] = acc;
      }
      // st was last read by X, Y (two barriers ago): safe to rewrite now
#pragma unroll
      for (int t = 0; t < STW; t++) {
        const int rb = (wave * STW + t) * 16;
        st_col4(&sm.st[c][rb + r0], S[t]);
      }
    }
  }

  // ---- final state
  if (a.state_out) {
    const int c = lane & 15, r0 = (lane >> 4) * 4;
    float* so = a.state_out + ((long)seq * a.hv + h) * DK * a.dv;
#pragma unroll
    for (int t = 0; t < STW; t++) {
      const int rb = (wave * STW + t) * 16;
#pragma unroll
      for (int e = 0; e < 4; e++) so[(long)(rb + r0 + e) * a.dv + dv0 + c] = S[t][e];
    }
  }
}

template <class E, int C, int DK>
hipError_t launch_prepare_t(const ScanArgs& a, hipStream_t s) {
  dim3 grid(a.max_chunks, a.hv), block(256);
  hipLaunchKernelGGL((k_prepare<E, C, DK>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <class E, int C, int DK>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  const int GS = (a.hv / a.hk) * (a.dv / 16);
  const int ngroups = a.num_seqs * a.hk;
  const int per_xcd = (ngroups + 7) / 8;
  dim3 grid(8 * per_xcd * GS), block(256);
  hipLaunchKernelGGL((k_scan<E, C, DK>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <class E, template <class, int, int> class F>
struct Dispatch;

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
  return a.dtype == 1 ? dispatch_scan<BF16>(a, s) : dispatch_scan<F32>(a, s);
}

}  // namespace gdn
