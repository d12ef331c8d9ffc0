/*
 * unroll.c -- the sequential unroll s_t = f(s_{t-1}, x_t) of the diagonal GRU
 * and LSTM cells in plain C, float64 arithmetic, parallel over independent
 * channels with OpenMP.
 *
 * Test infrastructure, like the rest of oracle/: the multi-core CPU baseline
 * the bench times, and a second, independent implementation of the NumPy
 * oracle's unroll (oracle/newton.py, sequential) that a CPU test compares
 * with it.  It shares no code with the HIP library.
 *
 * Cells (the diagonal "mix='diag'" cells of the shapes/layout page's support
 * table; the LSTM is the textbook one without peepholes, recurrent matrix
 * replaced by diag(a)), with x_* the projected inputs, biases included:
 *   GRU   z = sig(x_z + a_z h)  r = sig(x_r + a_r h)  c = tanh(x_c + a_c r h)
 *         h' = (1 - z) h + z c
 *   LSTM  i = sig(x_i + a_i h)  f = sig(x_f + a_f h)  o = sig(x_o + a_o h)
 *         g = tanh(x_g + a_g h)  c' = f c + i g       h' = o tanh(c')
 * Segment heads (row starts, and every cu_seqlens offset of a ragged pack,
 * shapes/layout page) restart from that segment's initial state.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static double sig(double u) { return 1.0 / (1.0 + exp(-u)); }

enum { CELL_GRU = 0, CELL_LSTM = 1 };
enum { BLOCK = 16 };   /* channels one OpenMP iteration walks side by side */

/*
 * xp   (B, T, G, d) float32: the stored projected inputs (read, then widened)
 * a    (G, d) float64 recurrent weights
 * h0   (rows, S, d) float64 initial states, or NULL for zeros (rows = B, or
 *      n_seqs for a ragged pack)
 * cu   NULL, or the (n_seqs + 1) offsets of a ragged pack (B = 1)
 * out  (B, T, d) float64: h_1 .. h_T of every row
 * Returns 0, or -1 on bad arguments.
 */
int oracle_unroll(int cell, int64_t B, int64_t T, int64_t d, const float* xp, const double* a, const double* h0,
                  int64_t n_seqs, const int32_t* cu, double* out) {
  const int G = cell == CELL_GRU ? 3 : 4, S = cell == CELL_GRU ? 1 : 2;
  if ((cell != CELL_GRU && cell != CELL_LSTM) || B < 1 || T < 0 || d < 1 || (cu && B != 1)) return -1;
  const int64_t n_blocks = (d + BLOCK - 1) / BLOCK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t job = 0; job < B * n_blocks; ++job) {
    const int64_t b = job / n_blocks, i0 = (job % n_blocks) * BLOCK;
    const int64_t n = (d - i0 < BLOCK) ? d - i0 : BLOCK;
    double c[BLOCK], h[BLOCK];
    int64_t seg = 0;  /* segment of the current step (ragged pack) */
    for (int64_t t = 0; t < T; ++t) {
      /* a head: row start, or the first step of a (non-empty) segment */
      int head = (t == 0);
      if (cu) {
        while (seg + 1 < n_seqs && cu[seg + 1] <= t) ++seg;
        if (cu[seg] == t) head = 1;
      }
      if (head) {
        const int64_t row = cu ? seg : b;
        for (int64_t k = 0; k < n; ++k) {
          c[k] = (h0 && S == 2) ? h0[(row * S + 0) * d + i0 + k] : 0.0;
          h[k] = h0 ? h0[(row * S + (S - 1)) * d + i0 + k] : 0.0;
        }
      }
      const float* x = xp + (b * T + t) * G * d + i0;
      double* o = out + (b * T + t) * d + i0;
      for (int64_t k = 0; k < n; ++k) {
        const int64_t i = i0 + k;
        if (cell == CELL_GRU) {
          const double z = sig((double)x[k] + a[i] * h[k]);
          const double r = sig((double)x[d + k] + a[d + i] * h[k]);
          const double cc = tanh((double)x[2 * d + k] + a[2 * d + i] * (r * h[k]));
          h[k] = (1.0 - z) * h[k] + z * cc;
        } else {
          const double ig = sig((double)x[k] + a[i] * h[k]);
          const double fg = sig((double)x[d + k] + a[d + i] * h[k]);
          const double og = sig((double)x[2 * d + k] + a[2 * d + i] * h[k]);
          const double gg = tanh((double)x[3 * d + k] + a[3 * d + i] * h[k]);
          c[k] = fg * c[k] + ig * gg;
          h[k] = og * tanh(c[k]);
        }
        o[k] = h[k];
      }
    }
  }
  return 0;
}
