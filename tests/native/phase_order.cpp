// CPU check of the phase kernels' tile order (combine_wave_level_amd/csrc/wave_sched.h:
// phase_xcd_order, phase_tiles, phase_tile), the same host+device functions the
// kernels call with blockIdx.x and gridDim.x.
//
// stdin: lines "BT NT grid E_local count_0 ... count_{E_local-1}" (expert row counts).
// For each case, over all workgroups of the grid and both orders (the plain one
// and the XCD-affine one): every (m-tile, n-tile) pair is run exactly once, by
// the expert that owns the m-tile; in the XCD-affine order on a grid that is a
// multiple of 8, workgroup b runs only positions of run b % 8, the runs have
// equal lengths (to within one), and the m-tiles of an expert that share an
// n-tile sit at adjacent list positions.  Prints "OK <cases>" (exit 0) or the
// first failure (exit 1).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../combine_wave_level_amd/csrc/wave_sched.h"

using namespace moe;

static int fail(const char* what, int c) {
  std::printf("FAIL case %d: %s\n", c, what);
  return 1;
}

int main() {
  int BT, NT, grid, E, ncase = 0;
  while (std::scanf("%d %d %d %d", &BT, &NT, &grid, &E) == 4) {
    std::vector<int32_t> mt_pre(E + 1, 0);
    for (int e = 0; e < E; ++e) {
      int c = 0;
      if (std::scanf("%d", &c) != 1) return fail("short input", ncase);
      mt_pre[e + 1] = mt_pre[e] + (c + BT - 1) / BT;
    }
    const int M = mt_pre[E], total = M * NT;
    for (int xo = 0; xo < 2; ++xo) {
      std::vector<int> seen(static_cast<size_t>(total), 0);
      std::vector<int> pos_of(static_cast<size_t>(total), -1);
      for (int b = 0; b < grid; ++b) {
        const PhaseTiles r = phase_tiles(total, xo != 0, b, grid);
        if (xo && grid % kXcds == 0) {
          const int x = b % kXcds;
          const long long lo = static_cast<long long>(total) * x / kXcds;
          const long long hi = static_cast<long long>(total) * (x + 1) / kXcds;
          if (r.begin != lo || r.end != hi) return fail("run bounds", ncase);
          if (hi - lo > total / kXcds + 1) return fail("run length", ncase);
        }
        for (int g = r.begin + r.first; g < r.end; g += r.stride) {
          int e = -1, mt = -1, nt = -1;
          phase_tile(mt_pre.data(), E, NT, g, xo != 0, e, mt, nt);
          if (e < 0 || e >= E || mt < mt_pre[e] || mt >= mt_pre[e + 1]) return fail("owner", ncase);
          if (nt < 0 || nt >= NT) return fail("n-tile range", ncase);
          const size_t id = static_cast<size_t>(mt) * NT + nt;
          if (seen[id]++) return fail("tile run twice", ncase);
          pos_of[id] = g;
        }
      }
      for (int i = 0; i < total; ++i)
        if (seen[static_cast<size_t>(i)] != 1) return fail("tile never run", ncase);
      if (xo) {
        // the m-tiles of one expert sharing an n-tile are adjacent in the list
        for (int e = 0; e < E; ++e)
          for (int mt = mt_pre[e] + 1; mt < mt_pre[e + 1]; ++mt)
            for (int nt = 0; nt < NT; ++nt)
              if (pos_of[static_cast<size_t>(mt) * NT + nt] != pos_of[static_cast<size_t>(mt - 1) * NT + nt] + 1)
                return fail("m-tiles of an n-tile not adjacent", ncase);
      }
    }
    ++ncase;
  }
  std::printf("OK %d\n", ncase);
  return 0;
}
