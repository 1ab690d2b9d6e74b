// Backward of the latent mixing steps between the down-projection and the
// attention (gfx950, HBM bound): causal sequence convolution, channel
// convolution, q-k-mean, value-shift, L2 normalisation and RoPE
// [GS-EN "2. Methodology" / Convolutional Mixing, Q-K-Mean, Value-Shift,
//  RoPE Integration; EDG "How Compressed Convolutional Attention Works"].
// Each step's derivative is the chain rule on the forward definition:
//   RoPE is a rotation per channel pair: its transpose rotates back;
//   y = m / max(|m|, eps):  dm = (dy - y <y, dy>) / |m| (|m| > eps), dy / eps;
//   q-k-mean (q += (q~ + k~_g) / 2, k += (k~ + mean_g q~) / 2): q~ collects
//     dq / 2 and dk_g / (2G), k~ collects dk / 2 and the group sum of dq / 2;
//   channel conv b[i] = sum_j w[j] a[i-j]:  da[i] = sum_j w[j] db[i+j];
//   sequence conv a[t] = sum_j w[j] u[t-j]: du[t] = sum_j w[j] da[t+j];
//   value-shift: the shifted heads' token t feeds token t+1.
//
// Design (MI355X): two passes over fp32 activations.
//  * head pass: d/4 lanes per (run of 8 tokens, q or k head), 4 channels per
//    lane, recompute the forward from the fp32 down-projection output
//    (sequence and channel conv, q-k-mean, norm, rotation) and run the
//    per-head backward (RoPE, norm, channel conv) token by token over the
//    run.  It writes dm (the mixed q/k cotangent) and da (the sequence conv
//    output's cotangent), plus per-(run, head) partial sums of the
//    channel-tap and temperature gradients.
//  * channel pass: one thread per (channel, 16-token run) combines the
//    sequence-conv transpose (reads da at t .. t+k_s-1), the q-k-mean skip
//    terms and the value-shift into dz, the cotangent of the down-projection
//    output, and accumulates its sequence-tap gradient over the run.
//  * tap / temperature gradients: deterministic two-level column sums.
#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

// Tokens per run of the head pass.
static constexpr int MIX_BWD_HTB = 8;

// Head-pass phases.  With the q-k-mean of the pre-convolution values only
// (or none) the channel conv's input cotangent is dm itself and one pass does
// everything (PH_ALL).  With the pre- and post-convolution mean, b_q of head h
// also reaches k of its group (and b_k every q head of the group), so
// db = 1.25 dm + (partner terms) needs the other heads' dm: PH_DM writes dm
// and the temperature partials, then PH_DA forms db from the dm of the head
// and its partners and runs the channel-conv transpose.
enum { PH_ALL = 0, PH_DM = 1, PH_DA = 2 };

template <typename TI, int D, int PH>
__global__ __launch_bounds__(256) void mix_bwd_head_kernel(MixShape s, MixTaps w,
                                                           const TI *__restrict__ qkv,
                                                           const float *__restrict__ bpost,
                                                           const float *__restrict__ gq,
                                                           const float *__restrict__ dk,
                                                           float *__restrict__ dm_io,
                                                           float *__restrict__ da_out,
                                                           float *__restrict__ tau_part,
                                                           float *__restrict__ chan_part) {
  // d/4 lanes per (run of MIX_BWD_HTB tokens, head), 4 consecutive channels
  // per lane (the layout of the forward mixing): the channel conv's
  // neighbours are one lane away, RoPE pairs stay in-lane, the norms are
  // d/4-lane reductions.  A lane group walks its run with a rolling window
  // of the k_s pre-conv rows, so every qkv row and tap is read once per run,
  // and the tap / temperature partials are summed over the run in registers.
  constexpr int LPU = D / 4;
  constexpr int UPW = 64 / LPU;             // units per wave (consecutive heads)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LPU;
  const int H = s.Hq + s.Hkv;
  const int ntb = (s.T + MIX_BWD_HTB - 1) / MIX_BWD_HTB;
  // the host keeps B * ntb * (Hq + Hkv) below 2^31
  const int unit = ((int)blockIdx.x * 4 + wave) * UPW + lane / LPU;
  const bool active = unit < s.B * ntb * H;
  const int run = active ? unit / H : 0;   // b * ntb + tb
  const int hh = active ? unit - run * H : 0;
  const int b = run / ntb, t0 = (run - b * ntb) * MIX_BWD_HTB;
  const int t1 = active ? min(s.T, t0 + MIX_BWD_HTB) : t0;
  const bool is_q = hh < s.Hq;
  const int g = is_q ? hh / s.G : hh - s.Hq;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int i0 = 4 * li;                                   // this lane's first channel
  const int colbase = is_q ? hh * D : eq + g * D;          // in the qkv row and in dm / da / b rows
  const int wcols = eq + ekv;
  const float *seqw = is_q ? w.q_seq + (size_t)hh * D * s.ks : w.k_seq + (size_t)g * D * s.ks;
  const float *chw = is_q ? w.q_chan + (size_t)hh * s.kc : w.k_chan + (size_t)g * s.kc;
  const TI *seq0 = qkv + (size_t)b * s.T * N;              // this sequence's rows
  const float *gin0 = is_q ? gq + (size_t)b * s.T * eq + hh * D + i0
                           : dk + (size_t)b * s.T * ekv + g * D + i0;
  const int gstride = is_q ? eq : ekv;
  // the q-k-mean: m = cb * b + coef * (own pre-conv + partner pre-conv +
  // partner post-conv); the post-conv partner term only in mean mode 2
  const bool post = s.use_mean == 2;
  const float cb = post ? 1.25f : 1.f, coef = post ? 0.25f : 0.5f;

  float ws[4][4];                                           // [channel][tap], zero past k_s
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) ws[c][j] = j < s.ks ? seqw[(i0 + c) * s.ks + j] : 0.f;
  float cw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cw[j] = j < s.kc ? chw[j] : 0.f;
  const double th0 = s.theta[li * 2], th1 = s.theta[li * 2 + 1];
  const float tau_h = is_q ? w.tau[hh] : 0.f;
  const float invg = __builtin_amdgcn_rcpf((float)s.G);

  // pre-conv row of token t (zero before the sequence start), the partner
  // sum of the q-k-mean (PH_ALL, PH_DM) or the partner cotangent of db
  // (PH_DA), and the incoming cotangent of token t (PH_ALL, PH_DM)
  auto load_row = [&](int t) -> f32x4 {
    if (t < 0) return f32x4{0.f, 0.f, 0.f, 0.f};
    return ld4f<TI>(seq0 + (size_t)t * N + colbase + i0);
  };
  auto load_skip = [&](int t) -> f32x4 {
    const size_t r = (size_t)b * s.T + t;
    if constexpr (PH == PH_DA) {
      // q head: dm of its key head / (4G); key head: the group's summed q dm / 4
      const float *row = dm_io + r * wcols;
      if (is_q) return *reinterpret_cast<const f32x4 *>(row + eq + g * D + i0) * (0.25f * invg);
      f32x4 m = *reinterpret_cast<const f32x4 *>(row + g * s.G * D + i0);
      for (int h2 = 1; h2 < s.G; ++h2) m += *reinterpret_cast<const f32x4 *>(row + (g * s.G + h2) * D + i0);
      return m * 0.25f;
    } else {
      const TI *row = seq0 + (size_t)t * N;
      f32x4 p;
      if (is_q) {
        p = ld4f<TI>(row + eq + g * D + i0);
        if (post) p += *reinterpret_cast<const f32x4 *>(bpost + r * wcols + eq + g * D + i0);
      } else {
        p = ld4f<TI>(row + g * s.G * D + i0);
        for (int h2 = 1; h2 < s.G; ++h2) p += ld4f<TI>(row + (g * s.G + h2) * D + i0);
        if (post)
          for (int h2 = 0; h2 < s.G; ++h2)
            p += *reinterpret_cast<const f32x4 *>(bpost + r * wcols + (g * s.G + h2) * D + i0);
        p = p * invg;
      }
      return p;
    }
  };
  auto load_gin = [&](int t) -> f32x4 {
    if constexpr (PH == PH_DA)
      return *reinterpret_cast<const f32x4 *>(dm_io + ((size_t)b * s.T + t) * wcols + colbase + i0);
    else
      return *reinterpret_cast<const f32x4 *>(gin0 + (size_t)t * gstride);
  };

  // lane exchanges: DPP inside rows of 16 lanes, shuffles across rows (d = 128)
  auto prev = [&](float v) {                               // value of the lane below (0 for li = 0)
    float r;
    if constexpr (LPU <= 16) r = dpp_shr1(v);
    else r = __shfl_up(v, 1, LPU);
    return li == 0 ? 0.f : r;
  };
  auto next = [&](float v) {                               // value of the lane above (0 for the last)
    float r;
    if constexpr (LPU <= 16) r = dpp_shl1(v);
    else r = __shfl_down(v, 1, LPU);
    return li == LPU - 1 ? 0.f : r;
  };
  auto grp_sum = [&](float v) { return group_sum<LPU>(v); };

  f32x4 u[4];                                               // rows t, t-1, t-2, t-3
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = load_row(t0 - j);
  const bool need_skip = PH == PH_DA || s.use_mean;
  f32x4 skip = need_skip ? load_skip(t0) : f32x4{0.f, 0.f, 0.f, 0.f}, gin = load_gin(t0);
  float tau_acc = 0.f, cacc[4] = {0.f, 0.f, 0.f, 0.f};

  // a uniform trip count keeps every lane in the wave-wide exchanges; tokens
  // past the run's end are computed on clamped rows and dropped
  for (int k = 0; k < MIX_BWD_HTB; ++k) {
    const int t = t0 + k;
    const bool valid = t < t1;
    // next token's inputs, in flight while this one is computed
    const int tn = min(t + 1, t1 - 1 < t0 ? t0 : t1 - 1);
    const f32x4 u_n = load_row(tn);
    const f32x4 skip_n = need_skip ? load_skip(tn) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 gin_n = load_gin(tn);

    // sequence conv of the pre-conv rows
    float a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(ws[c][j], u[j][c], acc);
      a[c] = acc;
    }
    const float p1 = prev(a[1]), p2 = prev(a[2]), p3 = prev(a[3]);   // a[i0-3], a[i0-2], a[i0-1]

    float dm[4];
    if constexpr (PH == PH_DA) {
      // db = 1.25 dm + the partners' terms
#pragma unroll
      for (int c = 0; c < 4; ++c) dm[c] = 1.25f * gin[c] + skip[c];
    } else {
      // forward recompute: channel conv, q-k-mean, norm
      float m[4];
      m[0] = cw[0] * a[0] + cw[1] * p3 + cw[2] * p2 + cw[3] * p1;
      m[1] = cw[0] * a[1] + cw[1] * a[0] + cw[2] * p3 + cw[3] * p2;
      m[2] = cw[0] * a[2] + cw[1] * a[1] + cw[2] * a[0] + cw[3] * p3;
      m[3] = cw[0] * a[3] + cw[1] * a[2] + cw[2] * a[1] + cw[3] * a[0];
      if (s.use_mean)
#pragma unroll
        for (int c = 0; c < 4; ++c) m[c] = cb * m[c] + coef * (u[0][c] + skip[c]);
      // 1 / max(||m||, eps) == rsqrt(max(||m||^2, eps^2))
      const float ss = grp_sum(m[0] * m[0] + m[1] * m[1] + m[2] * m[2] + m[3] * m[3]);
      const bool big = ss > s.eps * s.eps;
      const float inv = s.use_norm ? __builtin_amdgcn_rsqf(fmaxf(ss, s.eps * s.eps)) : 1.f;
      float n[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) n[c] = m[c] * inv;

      // RoPE pairs (i0, i0+1) and (i0+2, i0+3): rotate back, and the
      // temperature partial <r, g> of the rotated q
      float dn[4];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const float2 cs = rope_cs_theta(t, pp ? th1 : th0, s.rope_base);
        const float g0 = gin[2 * pp], g1 = gin[2 * pp + 1];
        const float d0 = is_q ? tau_h * g0 : g0, d1 = is_q ? tau_h * g1 : g1;
        const float x0 = n[2 * pp], x1 = n[2 * pp + 1];
        if (valid) tau_acc += (x0 * cs.x - x1 * cs.y) * g0 + (x0 * cs.y + x1 * cs.x) * g1;
        dn[2 * pp] = d0 * cs.x + d1 * cs.y;
        dn[2 * pp + 1] = -d0 * cs.y + d1 * cs.x;
      }

      // norm backward
      if (s.use_norm) {
        const float nd = grp_sum(n[0] * dn[0] + n[1] * dn[1] + n[2] * dn[2] + n[3] * dn[3]);
#pragma unroll
        for (int c = 0; c < 4; ++c) dm[c] = (big ? dn[c] - n[c] * nd : dn[c]) * inv;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) dm[c] = dn[c];
      }
      if (PH == PH_DM && valid) {
        const size_t o = ((size_t)b * s.T + t) * wcols + colbase + i0;
        *reinterpret_cast<f32x4 *>(dm_io + o) = f32x4{dm[0], dm[1], dm[2], dm[3]};
      }
    }

    if constexpr (PH != PH_DM) {
      // channel conv backward (da[i] = sum_j w_j db[i+j]) and its tap partials
      const float x0 = next(dm[0]), x1 = next(dm[1]), x2 = next(dm[2]);   // db[i0+4 .. i0+6]
      f32x4 da;
      da[0] = cw[0] * dm[0] + cw[1] * dm[1] + cw[2] * dm[2] + cw[3] * dm[3];
      da[1] = cw[0] * dm[1] + cw[1] * dm[2] + cw[2] * dm[3] + cw[3] * x0;
      da[2] = cw[0] * dm[2] + cw[1] * dm[3] + cw[2] * x0 + cw[3] * x1;
      da[3] = cw[0] * dm[3] + cw[1] * x0 + cw[2] * x1 + cw[3] * x2;
      if (valid) {
        cacc[0] += dm[0] * a[0] + dm[1] * a[1] + dm[2] * a[2] + dm[3] * a[3];
        cacc[1] += dm[0] * p3 + dm[1] * a[0] + dm[2] * a[1] + dm[3] * a[2];
        cacc[2] += dm[0] * p2 + dm[1] * p3 + dm[2] * a[0] + dm[3] * a[1];
        cacc[3] += dm[0] * p1 + dm[1] * p2 + dm[2] * p3 + dm[3] * a[0];
        const size_t o = ((size_t)b * s.T + t) * wcols + colbase + i0;
        if (PH == PH_ALL) *reinterpret_cast<f32x4 *>(dm_io + o) = f32x4{dm[0], dm[1], dm[2], dm[3]};
        *reinterpret_cast<f32x4 *>(da_out + o) = da;
      }
    }
    u[3] = u[2];
    u[2] = u[1];
    u[1] = u[0];
    u[0] = u_n;
    skip = skip_n;
    gin = gin_n;
  }

  if constexpr (PH != PH_DA) {
    const float tau_sum = grp_sum(tau_acc);
    if (active && li == 0 && is_q) tau_part[(size_t)run * s.Hq + hh] = tau_sum;
  }
  if constexpr (PH != PH_DM) {
    float cpart[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cpart[j] = grp_sum(cacc[j]);
    if (!active || li != 0) return;
    for (int j = 0; j < s.kc; ++j) chan_part[((size_t)run * H + hh) * s.kc + j] = cpart[j];
  }
}

// Tokens per thread of the channel pass.
static constexpr int MIX_BWD_TB = 16;

template <typename TI, typename TZ>
__global__ __launch_bounds__(256) void mix_bwd_chan_kernel(MixShape s, MixTaps w,
                                                           const TI *__restrict__ qkv,
                                                           const float *__restrict__ dm,
                                                           const float *__restrict__ da,
                                                           const float *__restrict__ dv,
                                                           TZ *__restrict__ dz,
                                                           float *__restrict__ seq_part) {
  const int D = s.d;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv, wcols = eq + ekv;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int ntb = (s.T + MIX_BWD_TB - 1) / MIX_BWD_TB;
  const int b = blockIdx.y / ntb, tb = blockIdx.y % ntb;
  const int tbeg = tb * MIX_BWD_TB, tend = min(s.T, tbeg + MIX_BWD_TB);
  if (c >= N) return;
  const size_t rb = (size_t)b * s.T;
  const float coef = s.use_mean == 2 ? 0.25f : 0.5f;
  if (c < wcols) {
    const bool is_q = c < eq;
    const int i = (is_q ? c : c - eq) % D;
    const int g = is_q ? (c / D) / s.G : (c - eq) / D;
    const float *seqw = is_q ? w.q_seq + (size_t)c * s.ks : w.k_seq + (size_t)(c - eq) * s.ks;
    float ws[4], dws[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ws[j] = j < s.ks ? seqw[j] : 0.f;
      dws[j] = 0.f;
    }
    // rolling windows: dwin[j] = da[t + j], uwin[j] = u[t - j] (zero outside [0, T))
    float dwin[4], uwin[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dwin[j] = (j < s.ks && tbeg + j < s.T) ? da[(rb + tbeg + j) * wcols + c] : 0.f;
      uwin[j] = (j < s.ks && tbeg - j >= 0) ? to_f32(qkv[(rb + tbeg - j) * N + c]) : 0.f;
    }
    for (int t = tbeg; t < tend; ++t) {
      const float nxt_d = (t + s.ks < s.T) ? da[(rb + t + s.ks) * wcols + c] : 0.f;
      const float nxt_u = (t + 1 < s.T) ? to_f32(qkv[(rb + t + 1) * N + c]) : 0.f;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += ws[j] * dwin[j];
      if (s.use_mean) {
        // the pre-conv values enter the mean with weight 1/2 (pre only) or
        // 1/4 (pre and post)
        const float *dmr = dm + (rb + t) * wcols;
        if (is_q) {
          acc += coef * dmr[c] + (coef / (float)s.G) * dmr[eq + g * D + i];
        } else {
          float qsum = 0.f;
          for (int h2 = 0; h2 < s.G; ++h2) qsum += dmr[(g * s.G + h2) * D + i];
          acc += coef * (dmr[c] + qsum);
        }
      }
      dz[(rb + t) * N + c] = from_f32<TZ>(acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) dws[j] += dwin[0] * uwin[j];
      // slide: window entries j >= ks stay zero (their taps are zero too)
#pragma unroll
      for (int j = 0; j < 3; ++j) dwin[j] = dwin[j + 1];
      dwin[3] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == s.ks - 1) dwin[j] = nxt_d;
#pragma unroll
      for (int j = 3; j > 0; --j) uwin[j] = uwin[j - 1];
      uwin[0] = nxt_u;
    }
    float *dst = seq_part + ((size_t)b * ntb + tb) * wcols * s.ks + (size_t)c * s.ks;
    for (int j = 0; j < s.ks; ++j) dst[j] = dws[j];
  } else {
    const int cv = c - wcols, gv = cv / D;
    const int shift = (s.use_shift && gv >= s.Hkv / 2) ? 1 : 0;
    for (int t = tbeg; t < tend; ++t) {
      const int src = t + shift;
      const float v = src < s.T ? dv[(rb + src) * ekv + cv] : 0.f;
      dz[(rb + t) * N + c] = from_f32<TZ>(v);
    }
  }
}

// Column sums of the per-row partials into the tap and temperature gradients.
// Each job sums columns col0 .. col0 + ncols of in [R][C] into out[ncols], in
// two launches for all jobs together: row blocks of COLSUM_ROWS rows into
// blk [nblk][ncols], then the block sums.  Fixed orders, so deterministic.
constexpr int COLSUM_ROWS = 64;
constexpr int COLSUM_JOBS = 5;
struct ColJob {
  const float *in;
  float *blk, *out;
  long long R;
  int C, col0, ncols, nblk;
};
struct ColJobs {
  ColJob j[COLSUM_JOBS];
  int first[COLSUM_JOBS + 1];   // first workgroup of each job in the row-block launch
};

// one workgroup per (job, row block, 64-column block), jobs back to back;
// 4 row phases of 16 rows each
__global__ __launch_bounds__(256) void colsum_rows_kernel(ColJobs jobs) {
  __shared__ float red[4][64];
  int z = 0;
  while (z + 1 < COLSUM_JOBS && (int)blockIdx.x >= jobs.first[z + 1]) ++z;
  const ColJob &jb = jobs.j[z];
  const int cb = (jb.ncols + 63) / 64;
  const int local = (int)blockIdx.x - jobs.first[z];
  const int bx = local % cb, by = local / cb;
  const int cl = threadIdx.x % 64, rs = threadIdx.x / 64;
  const int j = bx * 64 + cl;
  const long long r0 = (long long)by * COLSUM_ROWS;
  float v[COLSUM_ROWS / 4];
#pragma unroll
  for (int k = 0; k < COLSUM_ROWS / 4; ++k) {
    const long long r = r0 + rs + 4 * k;
    v[k] = (j < jb.ncols && r < jb.R) ? jb.in[r * jb.C + jb.col0 + j] : 0.f;
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < COLSUM_ROWS / 4; ++k) acc += v[k];
  red[rs][cl] = acc;
  __syncthreads();
  if (rs == 0 && j < jb.ncols)
    jb.blk[(size_t)by * jb.ncols + j] = (red[0][cl] + red[1][cl]) + (red[2][cl] + red[3][cl]);
}

// grid (64-column blocks, 1, jobs): the row-block sums, 4 row phases with
// four running sums each
__global__ __launch_bounds__(256) void colsum_blocks_kernel(ColJobs jobs) {
  __shared__ float red[4][64];
  const ColJob &jb = jobs.j[blockIdx.z];
  if ((int)blockIdx.x * 64 >= jb.ncols) return;
  const int cl = threadIdx.x % 64, rs = threadIdx.x / 64;
  const int j = blockIdx.x * 64 + cl;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (j < jb.ncols) {
    int r = rs;
    for (; r + 12 < jb.nblk; r += 16)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] += jb.blk[(size_t)(r + 4 * k) * jb.ncols + j];
    for (int k = 0; r < jb.nblk; r += 4, ++k) acc[k] += jb.blk[(size_t)r * jb.ncols + j];
  }
  red[rs][cl] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (rs == 0 && j < jb.ncols) jb.out[j] = (red[0][cl] + red[1][cl]) + (red[2][cl] + red[3][cl]);
}

static hipError_t colsum_all(ColJobs jobs, hipStream_t stream) {
  int cbmax = 1;
  jobs.first[0] = 0;
  for (int z = 0; z < COLSUM_JOBS; ++z) {
    const int cb = (jobs.j[z].ncols + 63) / 64;
    cbmax = max(cbmax, cb);
    jobs.first[z + 1] = jobs.first[z] + cb * jobs.j[z].nblk;
  }
  if (jobs.first[COLSUM_JOBS] > 0)
    hipLaunchKernelGGL(colsum_rows_kernel, dim3(jobs.first[COLSUM_JOBS]), dim3(256), 0, stream, jobs);
  hipLaunchKernelGGL(colsum_blocks_kernel, dim3(cbmax, 1, COLSUM_JOBS), dim3(256), 0, stream, jobs);
  return hipGetLastError();
}

static long long colsum_nblk(long long R) { return (R + COLSUM_ROWS - 1) / COLSUM_ROWS; }

size_t mix_backward_scratch_floats(const MixShape &s) {
  const size_t BR = (size_t)s.B * ((s.T + MIX_BWD_HTB - 1) / MIX_BWD_HTB);
  const int H = s.Hq + s.Hkv;
  const int ntb = (s.T + MIX_BWD_TB - 1) / MIX_BWD_TB;
  const size_t wcols = (size_t)(s.Hq + s.Hkv) * s.d;
  const size_t seq_rows = (size_t)s.B * ntb, seq_cols = wcols * s.ks;
  // tau partials, channel-tap partials (per head-pass run), seq-tap partials
  // (per channel-pass run), then the row-block sums of the five column sums
  // (each job its own)
  const size_t blk = colsum_nblk((long long)BR) * (size_t)(s.Hq + H * s.kc) +
                     colsum_nblk((long long)seq_rows) * seq_cols;
  return BR * s.Hq + BR * H * s.kc + seq_rows * seq_cols + blk;
}

template <typename TI, int D>
static hipError_t mix_bwd_heads(const MixShape &s, const MixTaps &w, const TI *qkv,
                                const float *bpost, const float *gq, const float *dk, float *dm,
                                float *da, float *tau_part, float *chan_part, unsigned nwg,
                                hipStream_t stream) {
  if (s.use_mean != 2) {
    hipLaunchKernelGGL((mix_bwd_head_kernel<TI, D, PH_ALL>), dim3(nwg), dim3(256), 0, stream, s, w,
                       qkv, bpost, gq, dk, dm, da, tau_part, chan_part);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((mix_bwd_head_kernel<TI, D, PH_DM>), dim3(nwg), dim3(256), 0, stream, s, w,
                     qkv, bpost, gq, dk, dm, da, tau_part, chan_part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mix_bwd_head_kernel<TI, D, PH_DA>), dim3(nwg), dim3(256), 0, stream, s, w,
                     qkv, bpost, gq, dk, dm, da, tau_part, chan_part);
  return hipGetLastError();
}

template <typename TI, typename TZ>
hipError_t launch_mix_backward(const MixShape &s, const MixTaps &w, const MixBwdArgs<TI, TZ> &a,
                               hipStream_t stream) {
  if (s.use_mean == 2 && !a.bpost) return hipErrorInvalidValue;
  const int nhr = (s.T + MIX_BWD_HTB - 1) / MIX_BWD_HTB;   // head-pass runs per sequence
  const long long units = (long long)s.B * nhr * (s.Hq + s.Hkv);
  const long long per_wg = 4LL * (64 / (s.d / 4));
  if (units + per_wg >= (1LL << 31)) return hipErrorInvalidValue;   // 32-bit unit indices
  const unsigned nwg = (unsigned)((units + per_wg - 1) / per_wg);
  const size_t BR = (size_t)s.B * nhr;
  const int H = s.Hq + s.Hkv;
  const int ntb = (s.T + MIX_BWD_TB - 1) / MIX_BWD_TB;
  const int wcols = (s.Hq + s.Hkv) * s.d, N = wcols + s.Hkv * s.d;
  const int eq = s.Hq * s.d, ekv = s.Hkv * s.d;
  float *tau_part = a.scratch;
  float *chan_part = tau_part + BR * s.Hq;
  float *seq_part = chan_part + BR * H * s.kc;
  float *blk = seq_part + (size_t)s.B * ntb * wcols * s.ks;

  hipError_t e;
  switch (s.d) {
    case 16: e = mix_bwd_heads<TI, 16>(s, w, a.qkv, a.bpost, a.gq, a.dk, a.dm, a.da, tau_part, chan_part, nwg, stream); break;
    case 32: e = mix_bwd_heads<TI, 32>(s, w, a.qkv, a.bpost, a.gq, a.dk, a.dm, a.da, tau_part, chan_part, nwg, stream); break;
    case 64: e = mix_bwd_heads<TI, 64>(s, w, a.qkv, a.bpost, a.gq, a.dk, a.dm, a.da, tau_part, chan_part, nwg, stream); break;
    case 128: e = mix_bwd_heads<TI, 128>(s, w, a.qkv, a.bpost, a.gq, a.dk, a.dm, a.da, tau_part, chan_part, nwg, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mix_bwd_chan_kernel<TI, TZ>), dim3((N + 255) / 256, s.B * ntb), dim3(256), 0,
                     stream, s, w, a.qkv, a.dm, a.da, a.dv, a.dz, seq_part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // temperature [B * nhr][Hq]; channel taps [B * nhr][H * kc] (q heads, then
  // k heads); sequence taps [B * ntb][(e_q + e_kv) * ks] (q channels, then k)
  const long long sr = (long long)s.B * ntb;
  const int nb_br = (int)colsum_nblk((long long)BR), nb_sr = (int)colsum_nblk(sr);
  ColJobs jobs;
  jobs.j[0] = ColJob{tau_part, blk, a.d_tau, (long long)BR, s.Hq, 0, s.Hq, nb_br};
  blk += (size_t)nb_br * s.Hq;
  jobs.j[1] = ColJob{chan_part, blk, a.d_q_chan, (long long)BR, H * s.kc, 0, s.Hq * s.kc, nb_br};
  blk += (size_t)nb_br * s.Hq * s.kc;
  jobs.j[2] = ColJob{chan_part, blk, a.d_k_chan, (long long)BR, H * s.kc, s.Hq * s.kc, s.Hkv * s.kc, nb_br};
  blk += (size_t)nb_br * s.Hkv * s.kc;
  jobs.j[3] = ColJob{seq_part, blk, a.d_q_seq, sr, wcols * s.ks, 0, eq * s.ks, nb_sr};
  blk += (size_t)nb_sr * eq * s.ks;
  jobs.j[4] = ColJob{seq_part, blk, a.d_k_seq, sr, wcols * s.ks, eq * s.ks, ekv * s.ks, nb_sr};
  return colsum_all(jobs, stream);
}

template hipError_t launch_mix_backward<f16, bf16>(const MixShape &, const MixTaps &,
                                                   const MixBwdArgs<f16, bf16> &, hipStream_t);
template hipError_t launch_mix_backward<float, float>(const MixShape &, const MixTaps &,
                                                      const MixBwdArgs<float, float> &, hipStream_t);

}  // namespace cca
