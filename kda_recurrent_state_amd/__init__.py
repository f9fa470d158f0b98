"""MI355X-native gated delta-rule (KDA / Gated DeltaNet) state layer."""
