"""CPU oracle for the CommunityKV decode step (test infrastructure only)."""
