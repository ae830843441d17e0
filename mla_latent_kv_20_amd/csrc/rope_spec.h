// RoPE frequency parameters shared by the host launchers and the kernels (plain data).
#pragma once

namespace mla {

// Pair k of a d-wide RoPE vector turns by theta^(-2k/d) per position ([notes] "MLA(Multi-head
// Latent Attention): DeepSeek-V2 논문정리", "MLA 코드 구현").  With yarn_s > 1 the
// frequencies follow YaRN's NTK-by-parts ([report] "Техотчёт DeepSeek-V2 (2024): MLA и
// экономика инференса", training and infrastructure section: each pair is scaled by how
// many turns it makes over the training length; DeepSeek-V2: s = 40, alpha = 1, beta = 32):
// a pair making r = L * f / (2 pi) turns over the training length L keeps f when r >= beta,
// becomes f / s when r <= alpha, and in between the linear blend
// (1 - g) f / s + g f with g = (r - alpha) / (beta - alpha).
struct RopeSpec {
  double log_theta;   // ln theta
  double yarn_s;      // scale factor s; <= 1: plain RoPE
  double yarn_len;    // training length L
  double yarn_alpha;
  double yarn_beta;
};

}  // namespace mla
