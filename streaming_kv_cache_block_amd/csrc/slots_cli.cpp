// slots_cli.cpp -- host-only driver of slots.h for the CPU tests (built with g++).
// Reads "S Ss W t1 t2 ..." lines on stdin: each line creates a fresh layer with S sink,
// Ss shot-sink and W window slots; a token n > 0 appends n frames, the token b starts
// a new shot.  After each append it prints one JSON object with f0, fs, the frame held
// by each slot, the slot runs of the cached context and the recache plans.
// A line "split B J n_cu" instead prints the split-walk plan of an attention launch of
// B blocks with J key tiles each on n_cu CUs (split_plan.h): whether it splits and the
// pieces every workgroup runs.
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "slots.h"
#include "split_plan.h"

static void print_plan(const char* name, const std::vector<ll::WriteEntry>& p) {
  std::cout << ",\"" << name << "\":[";
  for (size_t i = 0; i < p.size(); ++i)
    std::cout << (i ? "," : "") << "[" << p[i].src << "," << p[i].slot << "," << p[i].frame << "]";
  std::cout << "]";
}

static void print_split(std::istringstream& in) {
  int B = 0, J = 0, n_cu = 0;
  in >> B >> J >> n_cu;
  float dummy_ws = 0.0f;
  int dummy_cnt = 0;
  ll::Split sp{};
  sp.B = B;
  sp.J = J;
  sp.n_qtiles = 1;
  sp.ws = &dummy_ws;
  sp.cnt = &dummy_cnt;
  const bool on = ll::plan_split(sp, n_cu, ll::split_slots(n_cu));
  const int grid = on ? n_cu : (B + ll::kXcds - 1) / ll::kXcds * ll::kXcds;
  std::cout << "{\"B\":" << B << ",\"J\":" << J << ",\"n_cu\":" << n_cu << ",\"on\":" << (on ? 1 : 0)
            << ",\"slots\":" << ll::split_slots(n_cu) << ",\"pieces\":[";
  bool first = true;
  for (int wg = 0; wg < grid; ++wg)
    ll::for_each_piece(sp, wg, [&](const ll::Piece& p) {
      std::cout << (first ? "" : ",") << "[" << wg << "," << p.blk << "," << p.ja << "," << p.jb << "," << p.npc
                << "," << p.slot << "," << p.tail0 << "]";
      first = false;
    });
  std::cout << "]}\n";
}

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    if (line.rfind("split", 0) == 0) {
      std::string word;
      in >> word;
      print_split(in);
      continue;
    }
    ll::Layout L;
    if (!(in >> L.S >> L.Ss >> L.W)) continue;
    std::vector<int64_t> slot_frame(size_t(L.slots()), -1);
    int64_t f0 = 0, fs = 0;
    std::string tok;
    while (in >> tok) {
      if (tok == "b") {
        fs = f0;
        for (int s = L.S; s < L.S + L.Ss; ++s) slot_frame[size_t(s)] = -1;
        continue;
      }
      const int n = std::stoi(tok);
      for (const ll::WriteEntry& e : ll::append_plan(f0, n, L, fs)) slot_frame[size_t(e.slot)] = e.frame;
      f0 += n;
      std::cout << "{\"S\":" << L.S << ",\"Ss\":" << L.Ss << ",\"W\":" << L.W << ",\"f0\":" << f0 << ",\"fs\":" << fs
                << ",\"cached\":" << ll::cached_frames(f0, L, fs) << ",\"slot_frame\":[";
      for (size_t i = 0; i < slot_frame.size(); ++i) std::cout << (i ? "," : "") << slot_frame[i];
      std::cout << "],\"runs\":[";
      const std::vector<ll::SlotRun> runs = ll::cache_runs(f0, L, fs);
      for (size_t i = 0; i < runs.size(); ++i) std::cout << (i ? "," : "") << "[" << runs[i].first << "," << runs[i].count << "]";
      std::cout << "]";
      print_plan("recache", ll::recache_plan(f0, L, fs));
      print_plan("recache_window", ll::recache_window_plan(f0, L, fs));
      std::cout << "}\n";
    }
  }
  return 0;
}
