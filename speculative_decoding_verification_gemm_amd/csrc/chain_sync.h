// Counter arithmetic of the chain barrier (gemm_stream.hip), shared by the
// device code and host-side checks. Plain C++: no HIP types, so a host
// compiler can build it alone.
//
// Every counter is cumulative over launches of one prepared chain and is
// compared modulo 2^32; none is ever cleared between launches. With G
// workgroups per launch, after L complete launches:
//
//   gen              = L
//   exit_count       = L * G
//   group counter g  = L * gsize(g)     (per linear; gsize = workgroups in group g)
//   linear counter   = L * n_groups     (per linear)
//   release flags    = L * G            (per linear)
//
// A launch reads gen once and derives every target from gen1 = gen + 1, the
// launch count including itself. The products wrap modulo 2^32 exactly as
// the counters do, so equality tests stay exact across the wrap. (Deriving
// gen1 back from a wrapped product, as target / G, would not.)
#pragma once

#if defined(__HIP__)
#define SPECV_HD __host__ __device__
#else
#define SPECV_HD
#endif

namespace specv {

// Workgroups in arrival group g when G workgroups are dealt to `groups`
// groups by bid mod groups.
SPECV_HD inline unsigned chain_group_size(int G, int g, int groups) {
  return (unsigned)((G - g + groups - 1) / groups);
}

// The value the exit counter and the release flags reach in launch gen1.
SPECV_HD inline unsigned chain_target(unsigned gen1, int G) { return gen1 * (unsigned)G; }

// After an arrival bumped a group counter from `prev`: was it the group's
// last arrival in launch gen1?
SPECV_HD inline bool chain_group_complete(unsigned prev, unsigned gen1, unsigned gsize) {
  return prev + 1u == gen1 * gsize;
}

// After a group bumped a linear's counter from `prev`: was it the last
// group in launch gen1?
SPECV_HD inline bool chain_linear_complete(unsigned prev, unsigned gen1, int n_groups) {
  return prev + 1u == gen1 * (unsigned)n_groups;
}

// Has a release flag reached the target of this launch? Flags only move
// forward, by G per launch, so a wrapped difference tells earlier from later.
SPECV_HD inline bool chain_released(unsigned flag, unsigned target) {
  return (int)(flag - target) >= 0;
}

}  // namespace specv
