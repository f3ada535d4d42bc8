// Workgroup shape of the bf16 attention kernel: how many waves (W = 8, 4 or
// 2; a workgroup covers 32*W query rows of one (split, b, h)) a launch uses.
//
// Plain host C++ with no HIP types, so that a CPU test can compile it and
// check the choice for given shapes.
//
// Model.  A CU holds at most 8 waves of this kernel (two per SIMD, limited by
// registers), and the model lets it hold one 8-wave workgroup or up to two
// smaller ones at a time.  Workgroups are spread evenly, so the busiest CU
// gets n = ceil(workgroups / CUs) of them and runs them conc = min(n, cap) at
// a time in ceil(n / conc) rounds; a round moves conc * 32W query rows
// through the whole key range at a rate set by the waves the CU then holds.
// Relative rates, measured on MI355X at the FLUX-1024 shape (S = 4608,
// H = 24, D = 128) and at the ring-step share (576 x 576): 8 waves in one
// workgroup 1.0, in two 0.94; 4 waves 0.74; 2 waves 0.45.  Tiles past the
// last query row cost as much as full ones; the workgroup count includes
// them.
#pragma once

namespace cru {

inline double attn_wave_rate(int waves_on_cu, int w) {
  if (waves_on_cu >= 8) return w == 8 ? 1.0 : 0.94;
  if (waves_on_cu >= 4) return 0.74;
  return 0.45;
}

// row_blocks = splits * B * H; sq = query rows; n_cu = compute units.
inline int attn_pick_waves(long row_blocks, long sq, int n_cu) {
  const int ws[3] = {8, 4, 2};
  int best = 8;
  double best_cost = 0.0;
  for (int i = 0; i < 3; ++i) {
    const int w = ws[i];
    const int cap = w == 8 ? 1 : 2;
    const long rows = 32L * w;
    const long wgs = row_blocks * ((sq + rows - 1) / rows);
    const long n = (wgs + n_cu - 1) / n_cu;
    const long conc = n < cap ? n : cap;
    if (conc <= 0) return 8;   // empty launch: nothing runs
    const long rounds = (n + conc - 1) / conc;
    const double cost =
        (double)rounds * (double)(conc * rows) / attn_wave_rate((int)(conc * w), w);
    if (i == 0 || cost < best_cost) {
      best = w;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace cru
