// Host-side sweep of the library's planner for a sanitizer build: every call
// here is a host function (okls_default_config, okls_workspace_size,
// okls_plan_query, okls_ns_coefficients, okls_status_string), so no device is touched.  The
// planner lays out the workspace, builds the launch lists and checks every
// descriptor against its buffer; built with address and undefined-behaviour
// sanitizers on the host pass, this sweep makes any out-of-bounds access or
// undefined arithmetic in that code fail loudly.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../include/okls.h"

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 400;
  std::mt19937 rng(12345);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  long planned = 0, refused = 0;
  for (int r = 0; r < rounds; ++r) {
    okls_config c;
    okls_default_config(&c);
    c.mode = uni(0, 4);
    c.ns_steps = uni(2, 16);
    c.ns_split_steps = uni(0, 1) ? 0 : uni(0, c.ns_steps);
    c.factor_split = uni(0, 1);
    c.chunk_matrices = uni(0, 1) ? 0 : uni(1, 6);
    c.root_period = uni(1, 4);
    c.eps_convex = uni(0, 1);
    c.decay_after = uni(0, 1);
    c.shape_scale = uni(0, 1);
    c.ns_classical = uni(0, 1);
    c.whiten_split = uni(0, 1);
    c.soap_beta = 0.5f;
    c.precond_freq = uni(1, 4);
    c.soap_moments = uni(0, 1);
    c.bias_correction = uni(0, 1);
    c.jacobi_sweeps = uni(1, 3);
    c.nys_rank = uni(1, 40);
    c.nys_oversample = uni(0, 12);
    c.nys_passes = uni(0, 3);
    const int ng = uni(1, 16);
    std::vector<okls_group_desc> g(ng);
    for (okls_group_desc& d : g) {
      // mostly small sides, some large, some at the padding boundaries
      const int pick = uni(0, 9);
      auto side = [&]() {
        if (pick < 6) return uni(1, 300);
        if (pick < 8) return 128 * uni(1, 12) + uni(-1, 1);
        return uni(1, 3000);
      };
      d.batch = uni(1, 8);
      d.m = std::max(1, side());
      d.n = std::max(1, side());
      d.g_dtype = uni(0, 2);
    }
    const size_t ws = okls_workspace_size(&c, ng, g.data());
    if (ws == 0) ++refused; else ++planned;
    okls_plan_info info;
    const okls_status qs = okls_plan_query(&c, ng, g.data(), &info);
    if ((qs == OKLS_OK) != (ws != 0) ||
        (qs == OKLS_OK && (info.chunks < 1 || info.launches < 1 || info.ns_chains < 0 || info.ns_chains > 2))) {
      std::fprintf(stderr, "plan query disagrees with the workspace query\n");
      return 1;
    }
    double a[16], b[16];
    if (okls_ns_coefficients(&c, a, b, 16) != c.ns_steps) {
      std::fprintf(stderr, "coefficient table length mismatch\n");
      return 1;
    }
  }
  // invalid arguments: every one returns 0 / an error, never crashes
  okls_config c;
  okls_default_config(&c);
  okls_group_desc bad[17] = {};
  for (okls_group_desc& d : bad) d = okls_group_desc{1, 8, 8, 0};
  if (okls_workspace_size(&c, 17, bad) != 0 || okls_workspace_size(&c, 0, bad) != 0 ||
      okls_workspace_size(nullptr, 1, bad) != 0 || okls_workspace_size(&c, 1, nullptr) != 0) {
    std::fprintf(stderr, "an invalid argument was planned\n");
    return 1;
  }
  okls_group_desc big{1, 32768, 8, 0};
  if (okls_workspace_size(&c, 1, &big) == 0) {
    std::fprintf(stderr, "the largest side was refused\n");
    return 1;
  }
  for (int s = -8; s <= 1; ++s) (void)okls_status_string(static_cast<okls_status>(s));
  std::printf("planned %ld, refused %ld\n", planned, refused);
  return planned > 0 ? 0 : 1;
}
