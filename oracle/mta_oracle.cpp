// Multi-Token Attention forward: plain fp64 CPU oracle.
//
// TEST INFRASTRUCTURE ONLY. This file is the independent definition the GPU
// library is checked against. Only the test-suite, the smoke check and the
// benchmark's CPU-baseline leg may load it; the library never calls it and shares
// no code, header, table or helper with it.
//
// It evaluates the layer exactly as the page "Multi-Token Attention | Summary"
// (greeksharifa.github.io) states it, one step after another, in double precision,
// materialising every T x T map of one head group that the requested output rows
// need. There is no tiling, fusion or reordering beyond the definitions:
//
//   O1  logits  L = Q K^T / sqrt(d)                         (§2, attention logits)
//   O2  [mix pre]  L_u <- sum_u' w[u][u'] L_u'               (§3.2, the two-head
//                   mixing equations; mixing may act on logits, before softmax)
//   O3  [kq pre]   C = Conv2d_theta(Mask_0(L))               (§3.1, the pre-softmax
//                   equation; Mask_0 zeroes future keys per source row)
//   O4  Mask_-inf on j > i, row softmax                      (§2 causal mask; §3.1)
//   O5  [kq post]  C = Mask_0(Conv2d_theta(A))               (§3.1: the convolution
//                   may also act on the softmax weights, mixing them linearly)
//   O6  [mix post] A_u <- sum_u' w[u][u'] A_u'               (§3.2)
//   O7  O = A V                                              (§2, each head produces AV)
//   O8  [gn] per (token, head) GroupNorm over d, affine, times the gate value
//                                                            (§3.3, group normalisation
//                   and scalar gating before concatenation)
//
// Each of the two convolutions may act before softmax, after it, or on both sides
// (§4: unless stated otherwise the experiments apply them before and after softmax);
// a side has its own kernels. On one side both act in sequence, mixing first before
// softmax and the key-query convolution first after it (§3.3: together they form one
// convolution over queries, keys and the heads of a group).
//
// Readings of points the page leaves open (kept identical on the GPU side):
//   * theta[m][a][e] multiplies Z[i-a][j-(e-h0)], h0 = (c_k-1)/2: the query axis
//     only looks at current and past rows (§3.1), the key axis is centred.
//   * Positions outside [0,T) contribute value 0 (zero padding), also before softmax.
//   * Heads of group g are g*c_h .. g*c_h+c_h-1; w is w[group][out][in].
//   * GroupNorm: biased variance, eps = 1e-5, gamma/beta indexed [m*d + t];
//     out = lambda * (gamma * (O - mean) / sqrt(var + eps) + beta).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

struct Problem {
  const double* q;
  const double* k;
  const double* v;
  const double* theta_pre;   // [M][c_q][c_k], read if kq & PRE
  const double* theta_post;  // [M][c_q][c_k], read if kq & POST
  const double* w_pre;       // [M/c_h][c_h][c_h], read if mix & PRE
  const double* w_post;      // [M/c_h][c_h][c_h], read if mix & POST
  const double* gamma;       // [M*d]
  const double* beta;        // [M*d]
  double lambda;
  int B, T, M, d, c_q, c_k, c_h;
  int kq;   // bits: PRE (before softmax), POST (after softmax)
  int mix;  // bits: PRE, POST
  int gn;   // 0/1
};

constexpr int PRE = 1, POST = 2;

inline size_t idx4(const Problem& p, int b, int t, int m, int c) {
  return (((size_t)b * p.T + t) * p.M + m) * p.d + c;
}

// Per (b, group) working set: every map row that a requested output row needs.
struct GroupMaps {
  int T, c_h;
  std::vector<int> slot;        // global row -> slot of its logits, -1 if absent
  std::vector<int> rows;        // slot -> global row
  std::vector<double> logits;   // [slot][u][T]   logits after O1/O2
  std::vector<int> pslot;       // global row -> slot of its softmax row (kq post only)
  std::vector<int> prows;       // softmax slot -> global row
  std::vector<double> probs;    // [pslot][u][T]  softmax rows after O3/O4 (kq post only)
  double* L(int s, int u) { return &logits[((size_t)s * c_h + u) * T]; }
  double* P(int s, int u) { return &probs[((size_t)s * c_h + u) * T]; }
};

// O1 + O2 for one map row r of every head in group g.
void logits_row(const Problem& p, int b, int g, int r, GroupMaps& gm, int s) {
  const double scale = 1.0 / std::sqrt((double)p.d);
  std::vector<double> raw((size_t)p.c_h * p.T);
  for (int u = 0; u < p.c_h; ++u) {
    const int m = g * p.c_h + u;
    for (int j = 0; j < p.T; ++j) {
      double acc = 0.0;
      for (int c = 0; c < p.d; ++c) acc += p.q[idx4(p, b, r, m, c)] * p.k[idx4(p, b, j, m, c)];
      raw[(size_t)u * p.T + j] = acc * scale;
    }
  }
  for (int u = 0; u < p.c_h; ++u) {
    double* dst = gm.L(s, u);
    if (p.mix & PRE) {
      const double* wrow = p.w_pre + ((size_t)g * p.c_h + u) * p.c_h;
      for (int j = 0; j < p.T; ++j) {
        double acc = 0.0;
        for (int u2 = 0; u2 < p.c_h; ++u2) acc += wrow[u2] * raw[(size_t)u2 * p.T + j];
        dst[j] = acc;
      }
    } else {
      for (int j = 0; j < p.T; ++j) dst[j] = raw[(size_t)u * p.T + j];
    }
  }
}

// Mask_0 applied to the stored logits: the value at (r, s), or 0 if (r, s) is a
// future key (s > r) or lies outside the T x T map.
double masked_logit(GroupMaps& gm, int r, int s, int u) {
  if (r < 0 || s < 0 || s >= gm.T || s > r) return 0.0;
  return gm.L(gm.slot[r], u)[s];
}

// O4: causal row softmax of x[0..i] (entries j > i are -inf and get weight 0).
void causal_softmax(const double* x, int i, int T, double* out) {
  double mx = -std::numeric_limits<double>::infinity();
  for (int j = 0; j <= i; ++j) mx = std::max(mx, x[j]);
  double sum = 0.0;
  for (int j = 0; j <= i; ++j) {
    out[j] = std::exp(x[j] - mx);
    sum += out[j];
  }
  for (int j = 0; j <= i; ++j) out[j] /= sum;
  for (int j = i + 1; j < T; ++j) out[j] = 0.0;
}

// O3 + O4 for map row r of head u of group g: the softmax row, written to out[0..T).
void softmax_row(const Problem& p, int g, int r, int u, GroupMaps& gm, double* out) {
  const int T = p.T, h0 = (p.c_k - 1) / 2;
  if (p.kq & PRE) {
    // O3: C[r][j] = sum_a sum_e theta[a][e] * Z[r-a][j-e+h0]
    const double* th = p.theta_pre + (size_t)(g * p.c_h + u) * p.c_q * p.c_k;
    std::vector<double> row(T);
    for (int j = 0; j < T; ++j) {
      double acc = 0.0;
      for (int a = 0; a < p.c_q; ++a)
        for (int e = 0; e < p.c_k; ++e) acc += th[a * p.c_k + e] * masked_logit(gm, r - a, j - e + h0, u);
      row[j] = acc;
    }
    causal_softmax(row.data(), r, T, out);
  } else {
    causal_softmax(gm.L(gm.slot[r], u), r, T, out);
  }
}

// Softmax weight at (r, s) (zero outside the map), from the stored rows.
double prob_at(GroupMaps& gm, int r, int s, int u) {
  if (r < 0 || s < 0 || s >= gm.T) return 0.0;
  return gm.P(gm.pslot[r], u)[s];
}

// The attention row of output row i for every head of the group (after O3..O6).
void attention_row(const Problem& p, int g, int i, GroupMaps& gm, std::vector<double>& A) {
  const int T = p.T, c_h = p.c_h, h0 = (p.c_k - 1) / 2;
  A.assign((size_t)c_h * T, 0.0);
  for (int u = 0; u < c_h; ++u) {
    double* a_u = &A[(size_t)u * T];
    if (p.kq & POST) {
      // O5 on the softmax rows i-a: Mask_0 after the convolution.
      const double* th = p.theta_post + (size_t)(g * c_h + u) * p.c_q * p.c_k;
      for (int j = 0; j <= i; ++j) {
        double acc = 0.0;
        for (int a = 0; a < p.c_q; ++a)
          for (int e = 0; e < p.c_k; ++e) acc += th[a * p.c_k + e] * prob_at(gm, i - a, j - e + h0, u);
        a_u[j] = acc;
      }
    } else {
      softmax_row(p, g, i, u, gm, a_u);
    }
  }
  if (p.mix & POST) {
    // O6: A_u <- sum_u' w[u][u'] A_u'
    std::vector<double> mixed((size_t)c_h * T, 0.0);
    for (int u = 0; u < c_h; ++u) {
      const double* wrow = p.w_post + ((size_t)g * c_h + u) * c_h;
      for (int u2 = 0; u2 < c_h; ++u2)
        for (int j = 0; j < T; ++j) mixed[(size_t)u * T + j] += wrow[u2] * A[(size_t)u2 * T + j];
    }
    A.swap(mixed);
  }
}

// Adds row r (if inside the map and not present yet) to a row set.
void add_row(std::vector<int>& slot, std::vector<int>& rows, int r) {
  if (r >= 0 && slot[r] < 0) {
    slot[r] = (int)rows.size();
    rows.push_back(r);
  }
}

}  // namespace

extern "C" {

// Computes output rows of the layer in fp64.
//   q, k, v      [B, T, M, d] (row-major, token-major, heads concatenated)
//   kq, mix      placement bits: 1 before softmax, 2 after softmax, 3 both sides
//   theta        [n_kq, M, c_q, c_k], n_kq = number of kq bits; the kernels before
//                softmax come first (read when kq != 0)
//   w            [n_mix, M/c_h, c_h, c_h] (w[g][out][in]), before-softmax first
//                (read when mix != 0)
//   gamma, beta  [M*d]              (read when gn != 0)
//   out          [B, T, M, d]; only the requested rows of every batch are written
//   rows         list of query rows (NULL: every row), n_rows entries
//   maps         optional [B, M, n_rows_or_T, T] final attention rows (the weights
//                multiplied with V), or NULL
// Returns 0 on success, -1 on bad arguments.
int mta_oracle_forward(const double* q, const double* k, const double* v, const double* theta,
                       const double* w, const double* gamma, const double* beta, double lambda,
                       double* out, int B, int T, int M, int d, int c_q, int c_k, int c_h, int kq,
                       int mix, int gn, const int* rows, int n_rows, double* maps, int n_threads) {
  if (B <= 0 || T <= 0 || M <= 0 || d <= 0 || c_h <= 0 || M % c_h != 0) return -1;
  if (kq != 0 && (c_q <= 0 || c_k <= 0 || (c_k % 2) == 0)) return -1;
  if (kq == 0) c_q = c_k = 1;
  if (kq < 0 || kq > 3 || mix < 0 || mix > 3) return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  const size_t th_size = (size_t)M * c_q * c_k, w_size = (size_t)M * c_h;
  const double* theta_post = (kq == 3) ? theta + th_size : theta;
  const double* w_post = (mix == 3) ? w + w_size : w;
  Problem p{q, k, v, theta, theta_post, w, w_post, gamma, beta, lambda, B, T, M, d, c_q, c_k, c_h, kq, mix, gn};
  std::vector<int> out_rows;
  if (rows == nullptr) {
    for (int i = 0; i < T; ++i) out_rows.push_back(i);
  } else {
    for (int n = 0; n < n_rows; ++n) {
      if (rows[n] < 0 || rows[n] >= T) return -1;
      out_rows.push_back(rows[n]);
    }
  }
  const int n_out = (int)out_rows.size();
  // softmax rows that output row i needs: i-c_q+1 .. i after a post-softmax
  // convolution, else i; logit rows that softmax row r needs: r-c_q+1 .. r after a
  // pre-softmax convolution, else r
  const int post_lag = (kq & POST) ? c_q : 1;
  const int pre_lag = (kq & PRE) ? c_q : 1;

  for (int b = 0; b < B; ++b) {
    for (int g = 0; g < M / c_h; ++g) {
      GroupMaps gm;
      gm.T = T;
      gm.c_h = c_h;
      gm.slot.assign(T, -1);
      gm.pslot.assign(T, -1);
      std::vector<int> srows, sslot(T, -1);
      for (int i : out_rows)
        for (int a = 0; a < post_lag; ++a) add_row(sslot, srows, i - a);
      for (int r : srows)
        for (int a = 0; a < pre_lag; ++a) add_row(gm.slot, gm.rows, r - a);
      const int n_slots = (int)gm.rows.size();
      gm.logits.assign((size_t)n_slots * c_h * T, 0.0);
#pragma omp parallel for schedule(dynamic, 1)
      for (int s = 0; s < n_slots; ++s) logits_row(p, b, g, gm.rows[s], gm, s);
      if (kq & POST) {
        gm.prows = srows;
        gm.pslot = sslot;
        const int n_p = (int)srows.size();
        gm.probs.assign((size_t)n_p * c_h * T, 0.0);
#pragma omp parallel for schedule(dynamic, 1)
        for (int s = 0; s < n_p; ++s)
          for (int u = 0; u < c_h; ++u) softmax_row(p, g, srows[s], u, gm, gm.P(s, u));
      }
#pragma omp parallel for schedule(dynamic, 1)
      for (int n = 0; n < n_out; ++n) {
        const int i = out_rows[n];
        std::vector<double> A;
        attention_row(p, g, i, gm, A);
        std::vector<double> o(d);
        for (int u = 0; u < c_h; ++u) {
          const int m = g * c_h + u;
          const double* a_u = &A[(size_t)u * T];
          if (maps != nullptr) {
            double* dst = maps + (((size_t)b * M + m) * n_out + n) * T;
            std::memcpy(dst, a_u, sizeof(double) * T);
          }
          // O7: O = sum_j A[i][j] v_j; A[i][j] is exactly 0 for j > i (causal mask,
          // or Mask_0 after a post-softmax convolution), so the sum stops at j = i.
          for (int c = 0; c < d; ++c) o[c] = 0.0;
          for (int j = 0; j <= i; ++j)
            for (int c = 0; c < d; ++c) o[c] += a_u[j] * p.v[idx4(p, b, j, m, c)];
          double* dst = out + idx4(p, b, i, m, 0);
          if (gn) {
            // O8: GroupNorm over the d channels of (b, i, m), then the gate.
            double mean = 0.0;
            for (int c = 0; c < d; ++c) mean += o[c];
            mean /= d;
            double var = 0.0;
            for (int c = 0; c < d; ++c) var += (o[c] - mean) * (o[c] - mean);
            var /= d;
            const double inv = 1.0 / std::sqrt(var + 1e-5);
            for (int c = 0; c < d; ++c)
              dst[c] = lambda * (gamma[(size_t)m * d + c] * (o[c] - mean) * inv + beta[(size_t)m * d + c]);
          } else {
            for (int c = 0; c < d; ++c) dst[c] = o[c];
          }
        }
      }
    }
  }
  return 0;
}

int mta_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
